// The MFMA K loop shared by the three contractions of the search (direct loss, X^T X, and the
// Gram-form loss): a 256 x 256 fp32 tile of A B^T accumulated over K, where A and B are two
// row-major fp16 panels of 256 rows whose reduction index runs along the row.
//
// gfx950 design:
//   * 256 threads = 4 waves (2 x 2), workgroup tile 256 x 256, wave tile 128 x 128, BK = 32;
//   * v_mfma_f32_32x32x16_f16: 4 x 4 MFMA blocks per wave, 256 fp32 accumulators per lane
//     (held in AGPRs; one wave per SIMD);
//   * operands go from HBM straight into LDS (buffer_load_dwordx4 ... lds): no staging
//     registers and no ds_write; each wave instruction fills 1 KiB = 16 rows x 64 bytes. The
//     buffer range of each operand panel ends at its last valid row, so rows of a ragged tile
//     read as zeros without branches;
//   * four LDS stages of 32 KiB: the loads of steps k+1..k+4 are in flight while step k
//     computes (one stage ahead left the waves waiting ~40% of the time on loads whose lines
//     missed L2; with four, dropping the wait for them saves nothing: they land in time; LDS
//     bank conflicts: none). Fragment reads of the next step overlap the second half of the
//     current step's MFMAs; a stage's refill is split over two half steps, and every load
//     address is scalar arithmetic plus one per-lane offset (no vector ALU work per load);
//   * LDS layout: row r holds its 4 chunks of 16 bytes at positions c ^ f(r),
//     f(r) = ((r >> 1) & 3) ^ ((r >> 3) & 1), so the 128-bit fragment reads of 8 (and of 16)
//     consecutive rows at one chunk touch distinct banks whether the LDS has 32 or 64 banks.
//
// Accumulator layout (v_mfma_f32_32x32x16_f16): acc[i][j][e] of lane l holds the tile element
//   A row  wm * 128 + 32 i + 8 (e / 4) + 4 (l / 32) + e % 4,
//   B row  wn * 128 + 32 j + l % 32,
// with wave w = 2 wm + wn.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace awq {
namespace kloop {

constexpr int BM = kLossBM, BN = kLossBN, BK = kLossBK;
constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kRowBytes = BK * 2;                           // 64 bytes of a row per K step
constexpr int kStageBytes = (BM + BN) * kRowBytes;          // 32 KiB per stage
constexpr int kSmemBytes = kStages * kStageBytes;           // 128 KiB
constexpr int kRowsPerWave = BM / 4;                        // rows each wave loads per operand
constexpr int kRowsPerInst = 1024 / kRowBytes;              // 16 rows per 1 KiB wave load
constexpr int kInstPerOp = kRowsPerWave / kRowsPerInst;     // 4 loads per operand per step

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// s_waitcnt immediate that waits until at most n vector-memory loads are outstanding (gfx9
// encoding: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

// The K loop over four LDS stages (LDS addresses base + stage * kStageBytes, stage = kt % 4).
//
// Per step kt: the 16 MFMAs of the first half (k 0..15) with the reads of the second-half
// fragments and the second half of the refill of stage kt-1 (step kt+3) in between; wait until
// step kt+1 has landed (steps kt+2, kt+3 may still be in flight) and this wave's LDS reads are
// done; barrier; the 16 MFMAs of the second half with the first half of the refill of stage kt
// (step kt+4) and the reads of step kt+1's first-half fragments in between. The refill of a
// stage is split over two half steps so that both halves issue twelve memory instructions, one
// after each MFMA but every fourth. The instruction stream is laid out by hand (sched_barrier
// stops the scheduler from regrouping it): each MFMA keeps the matrix core busy for 32 cycles
// while the following load or LDS read issues.
struct Tile {
  rsrc_t ra, rb;        // operand panels
  uint32_t voff;        // this lane's byte offset inside a 16-row load slice (per lane)
  uint32_t soff;        // byte offset of this wave's first row (wave-uniform)
  uint32_t row_stride;  // bytes between rows
  uint32_t lds0;        // LDS address of stage 0 (wave-uniform)
  uint32_t rd[2][2];    // this lane's fragment read offsets in a stage: [operand][k half]
  int wave;             // wave-uniform
};

struct Frags {
  half8_t a[2][4], b[2][4];   // [k half][row block]
};

// Lane-dependent parts of a tile: load offsets and fragment read offsets. `row_stride` is the
// byte distance between consecutive rows of both panels.
__device__ __forceinline__ void tile_setup(Tile& T, const char* smem, uint32_t row_stride) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index and the LDS base are uniform: in scalar registers, every load address of
  // the loop below is scalar arithmetic plus the one per-lane offset
  T.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T.lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // lane l of load slice j fills LDS row wave*64 + 16j + l/4, physical chunk l%4, i.e. the
  // logical chunk (l%4) ^ swz(row); swz depends on row % 16 = l/4 only.
  const int lrow = lane >> 2;
  T.row_stride = row_stride;
  T.voff = (uint32_t)lrow * row_stride + (uint32_t)(((lane & 3) ^ swz(lrow)) * 16);
  T.soff = (uint32_t)(T.wave * kRowsPerWave) * row_stride;
  // fragment reads: lane l reads row (wave block) + 32 i + l%32 at chunk 2h + l/32; the
  // swizzle of a row does not change with the +32 i block offset, so one offset per (operand,
  // k half) serves all four row blocks.
  const int frow = lane & 31, fhalf = lane >> 5;
  const int wm = T.wave >> 1, wn = T.wave & 1;
  const int ra0 = wm * 128 + frow, rb0 = wn * 128 + frow;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    T.rd[0][h] = (uint32_t)(ra0 * kRowBytes + (((2 * h + fhalf) ^ swz(ra0)) << 4));
    T.rd[1][h] = (uint32_t)(BM * kRowBytes + rb0 * kRowBytes + (((2 * h + fhalf) ^ swz(rb0)) << 4));
  }
}

// Fragment i (i < 4: A row block i, else B row block i - 4) of k half h from stage `st`.
__device__ __forceinline__ void kl_read(const char* smem, const Tile& T, int st, int h, int i,
                                        Frags& F) {
  const char* base = smem + st * kStageBytes;
  if (i < 4)
    F.a[h][i] = *reinterpret_cast<const half8_t*>(base + T.rd[0][h] + i * 32 * kRowBytes);
  else
    F.b[h][i - 4] = *reinterpret_cast<const half8_t*>(base + T.rd[1][h] + (i - 4) * 32 * kRowBytes);
}

// Load slice idx in [0, 8) of step kt into stage `st` (even idx: A, odd: B; rows 16 (idx/2) ..
// of this wave's 64 rows).
__device__ __forceinline__ void kl_issue(const Tile& T, int st, int kt, int idx) {
  const int j = idx >> 1;
  const uint32_t lds = T.lds0 + (uint32_t)(st * kStageBytes) + ((idx & 1) ? BM * kRowBytes : 0) +
                       (uint32_t)((T.wave * kRowsPerWave + kRowsPerInst * j) * kRowBytes);
  const uint32_t so = T.soff + (uint32_t)(kRowsPerInst * j) * T.row_stride +
                      (uint32_t)kt * (uint32_t)kRowBytes;
  buffer_load16_lds_so((idx & 1) ? T.rb : T.ra, lds, T.voff, so);
}

// Load slice j in [0, 4) of operand A's rows of step `ksrc` into the B half of stage `st`, at
// the rows and chunk positions the A half uses (so the A fragment offsets read it back).
__device__ __forceinline__ void kl_issue_a_to_b(const Tile& T, int st, int ksrc, int j) {
  const uint32_t lds = T.lds0 + (uint32_t)(st * kStageBytes) + BM * kRowBytes +
                       (uint32_t)((T.wave * kRowsPerWave + kRowsPerInst * j) * kRowBytes);
  const uint32_t so = T.soff + (uint32_t)(kRowsPerInst * j) * T.row_stride +
                      (uint32_t)ksrc * (uint32_t)kRowBytes;
  buffer_load16_lds_so(T.ra, lds, T.voff, so);
}

// ------------------------------------------------------------------------------------------
// K-blocked operands: a panel stored as [K / 32][rows][32], so that the 256 x 32 tile of one K
// step is a contiguous 16 KiB block (rows 64 bytes apart). Each load takes a buffer descriptor
// built for its step: base + kt * (bytes between K blocks), range = the panel's valid rows x 64
// bytes, so rows past the panel read as zeros and no offset is limited to 32 bits. The LDS
// layout, and so every fragment read, is that of Tile (row_stride = 64 in tile_setup).
struct TileK : Tile {
  const char* pa;    // operand A: panel's first row in K block 0
  const char* pb;    // operand B
  uint64_t ka, kb;   // bytes between consecutive K blocks
  uint32_t na, nb;   // valid rows x 64 bytes
  int nkb;           // K blocks that exist: steps from nkb on read zeros (an empty range)
};

// TileK's operand B (the output columns) is interleaved between the two column waves: column
// half wn takes the 32-column blocks c = 2 j + wn (Tile: c = 4 wn + j), so that the two halves
// hold equal shares of the diagonal block of a lower-triangular B (kl_block_live below).
__device__ __forceinline__ void tile_setup_k(TileK& T, const char* smem) {
  tile_setup(T, smem, (uint32_t)kRowBytes);
  // B rows 32 wn + l % 32 instead of 128 wn + l % 32: the swizzle depends on bits 1..3 of the row
  // only, so the offsets just move
  const uint32_t d = (uint32_t)((T.wave & 1) * 96 * kRowBytes);
  T.rd[1][0] -= d;
  T.rd[1][1] -= d;
}

__device__ __forceinline__ void kl_read(const char* smem, const TileK& T, int st, int h, int i,
                                        Frags& F) {
  const char* base = smem + st * kStageBytes;
  if (i < 4)
    F.a[h][i] = *reinterpret_cast<const half8_t*>(base + T.rd[0][h] + i * 32 * kRowBytes);
  else
    F.b[h][i - 4] = *reinterpret_cast<const half8_t*>(base + T.rd[1][h] + (i - 4) * 64 * kRowBytes);
}

__device__ __forceinline__ void kl_issue(const TileK& T, int st, int kt, int idx) {
  const int j = idx >> 1;
  const bool b = idx & 1;
  const uint32_t live = kt < T.nkb ? 1u : 0u;
  const rsrc_t r = b ? make_rsrc(T.pb + (uint64_t)kt * T.kb, T.nb * live)
                     : make_rsrc(T.pa + (uint64_t)kt * T.ka, T.na * live);
  const uint32_t lds = T.lds0 + (uint32_t)(st * kStageBytes) + (b ? BM * kRowBytes : 0) +
                       (uint32_t)((T.wave * kRowsPerWave + kRowsPerInst * j) * kRowBytes);
  buffer_load16_lds_so(r, lds, T.voff, T.soff + (uint32_t)(kRowsPerInst * j) * T.row_stride);
}

__device__ __forceinline__ void kl_issue_a_to_b(const TileK& T, int st, int ksrc, int j) {
  const uint32_t lds = T.lds0 + (uint32_t)(st * kStageBytes) + BM * kRowBytes +
                       (uint32_t)((T.wave * kRowsPerWave + kRowsPerInst * j) * kRowBytes);
  buffer_load16_lds_so(make_rsrc(T.pa + (uint64_t)ksrc * T.ka, ksrc < T.nkb ? T.na : 0u), lds,
                       T.voff,
                       T.soff + (uint32_t)(kRowsPerInst * j) * T.row_stride);
}

// LO: issue loads 0..3 of step kt+4 (into stage kt); HI: issue loads 4..7 of step kt+3 (into
// stage kt-1, free since the barrier of step kt-1); MORE: read step kt+1's first-half fragments;
// VM: loads allowed in flight at the wait (those issued after the last load of step kt+1);
// COPY: in the slots of LO, load operand A of step kt-4 into the B half of stage kt (free after
// this step's barrier), for an epilogue that reads A of the last eight steps.
// KD >= 0: step KD of the last eight, which cover the diagonal 256 x 256 block of a B that is
// lower triangular (B[l][k] = 0 for k > l, l and k counted from the tile's first column): the
// products of block j of wave column half wn have k >= 32 KD and l < 128 wn + 32 (j + 1), so
// they are all zero when KD > 4 wn + j, and those MFMAs are skipped (the loads and fragment reads
// stay as they are).
__device__ __forceinline__ bool kl_block_live(int KD, int j, const Tile& T) {
  return KD < 0 || KD <= j || (KD - 4 <= j && (T.wave & 1));
}
// the same with TileK's interleaved columns (block j of column half wn is c = 2 j + wn): zero
// when KD > 2 j + wn
__device__ __forceinline__ bool kl_block_live(int KD, int j, const TileK& T) {
  return KD < 0 || KD <= 2 * j || (KD == 2 * j + 1 && (T.wave & 1));
}

template <bool LO, bool HI, bool MORE, int VM, bool COPY = false, int KD = -1, class TT = Tile>
__device__ __forceinline__ void kl_step(const char* smem, const TT& T, int kt, Frags& F,
                                        floatx16 (&acc)[4][4]) {
  const int st = kt & 3;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (kl_block_live(KD, m & 3, T))
      acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[0][m >> 2], F.b[0][m & 3],
                                                                  acc[m >> 2][m & 3], 0, 0, 0);
    if ((m & 1) == 0) kl_read(smem, T, st, 1, m >> 1, F);
    if (HI && (m & 3) == 1) kl_issue(T, (st + 3) & 3, kt + 3, 4 + (m >> 2));
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt(VM) & ~0x0F00);   // + lgkmcnt(0)
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (kl_block_live(KD, m & 3, T))
      acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[1][m >> 2], F.b[1][m & 3],
                                                                  acc[m >> 2][m & 3], 0, 0, 0);
    if (LO && (m & 3) == 0) kl_issue(T, st, kt + 4, m >> 2);
    if (COPY && (m & 3) == 0) kl_issue_a_to_b(T, st, kt - 4, m >> 2);
    if (MORE && (m & 1)) kl_read(smem, T, (st + 1) & 3, 0, m >> 1, F);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc += A B^T over nk steps of BK (nk >= 4; nk >= 8 with COPY). The LDS stages must be free on
// entry (a barrier after any previous use); on return every wave has passed the last step's
// barrier and the stages are no longer read. With COPY, on return (once vmcnt(0) and a barrier
// have followed) stage s holds operand A of step nk-8+s in its B half and of step nk-4+s in its
// A half, s = 0..3 -- when nk is a multiple of 4 -- i.e. A of the last eight steps.
// TRI (nk >= 8): the last eight steps are the diagonal block of a lower-triangular B (kl_step's
// KD); their all-zero MFMA blocks are skipped.
template <bool COPY, bool TRI = false, class TT = Tile>
__device__ __forceinline__ void kl_run_t(const char* smem, const TT& T, int nk,
                                         floatx16 (&acc)[4][4]) {
  Frags F;
  // steps 0..2 in full, loads 0..3 of step 3 (its loads 4..7 follow in step 0)
#pragma unroll
  for (int p = 0; p < kStages; ++p)
#pragma unroll
    for (int idx = 0; idx < ((p < kStages - 1) ? 2 * kInstPerOp : kInstPerOp); ++idx)
      kl_issue(T, p, p, idx);
  __builtin_amdgcn_s_waitcnt(vmcnt(20));           // step 0 has landed
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) kl_read(smem, T, 0, 0, i, F);
  // at the wait of step kt, the loads of steps kt+2 and kt+3 (16) may be in flight
  for (int kt = 0; kt < nk - (TRI ? 8 : 4); ++kt)
    kl_step<true, true, true, 16, false, -1, TT>(smem, T, kt, F, acc);
  if constexpr (TRI) {
    kl_step<true, true, true, 16, false, 0, TT>(smem, T, nk - 8, F, acc);
    kl_step<true, true, true, 16, false, 1, TT>(smem, T, nk - 7, F, acc);
    kl_step<true, true, true, 16, false, 2, TT>(smem, T, nk - 6, F, acc);
    kl_step<true, true, true, 16, false, 3, TT>(smem, T, nk - 5, F, acc);
  }
  // the copies (4 per step, from step nk-4 on) come after the last loads of steps nk-1
  kl_step<false, true, true, 16, COPY, TRI ? 4 : -1, TT>(smem, T, nk - 4, F, acc);
  kl_step<false, false, true, COPY ? 12 : 8, COPY, TRI ? 5 : -1, TT>(smem, T, nk - 3, F, acc);
  kl_step<false, false, true, COPY ? 8 : 0, COPY, TRI ? 6 : -1, TT>(smem, T, nk - 2, F, acc);
  kl_step<false, false, false, COPY ? 12 : 0, COPY, TRI ? 7 : -1, TT>(smem, T, nk - 1, F, acc);
}

template <class TT>
__device__ __forceinline__ void kl_run(const char* smem, const TT& T, int nk,
                                       floatx16 (&acc)[4][4]) {
  kl_run_t<false, false, TT>(smem, T, nk, acc);
}

// ------------------------------------------------------------------------------------------
// The same K loop on operands stored with the reduction index across rows: X itself, [tokens]
// [channels] row-major, for X^T X without a transposed copy. A stage holds, per operand, BK = 32
// token rows of the panel's 256 channels (512 bytes each, 16 KiB); the fragment a lane needs (8
// consecutive tokens of one channel) is gathered by two ds_read_b64_tr_b16.
//
// ds_read_b64_tr_b16 (measured on gfx950): within each group of 16 lanes, lane 4 q + r receives,
// as its element j = 0..3, element r of the 64-bit word that lane 4 j + q addressed. So if lane
// 4 j + q addresses tokens t0 + j, channels c0 + 4 q .. c0 + 4 q + 3, lane L receives tokens
// t0 .. t0 + 3 of channel c0 + L: the MFMA operand layout (row = lane, four k values).
//
// LDS layout of a token row R: its 32 chunks of 8 channels, chunk c at position
// 4 ((c / 4) ^ (R % 4)) + c % 4. The 16 lanes of a half-wave read 4 token rows (R % 4 all
// different) x 4 chunks c0/8 .. c0/8 + 3 (c0 a multiple of 32): 16 distinct positions modulo
// 16, i.e. all 64 banks, once each.
struct TileX {
  rsrc_t ra, rb;        // operand panels: row t = token t of the chunk, 256 channels
  uint32_t voff[2];     // load lane offsets for slices of even / odd j (the swizzle key alternates)
  uint32_t soff;        // byte offset of this wave's first token row (wave-uniform)
  uint32_t row_stride;  // bytes between token rows
  uint32_t lds0;
  uint32_t rd[2][4];    // fragment read offsets in a stage: [operand][row block], k half 0
  int wave;
};

constexpr int kXRowBytes = BM * 2;   // 512 bytes: one token row of a 256-channel panel

__device__ __forceinline__ void tile_setup_x(TileX& T, const char* smem, uint32_t row_stride) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  T.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  T.lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  T.row_stride = row_stride;
  // load slice j of a wave fills token rows 8 wave + 2 j + lane / 32 (two per 1 KiB load);
  // lane l writes physical chunk l % 32, i.e. the logical chunk 4 ((p / 4) ^ (R % 4)) + p % 4
  const int p = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    const int rk = (2 * jp + hi) & 3;
    const int c = 4 * ((p >> 2) ^ rk) + (p & 3);
    T.voff[jp] = (uint32_t)hi * row_stride + (uint32_t)(c * 16);
  }
  T.soff = (uint32_t)(T.wave * 8) * row_stride;
  // fragment reads: lane l = 16 G' + L (G' = l / 16), L = 4 j' + q'. Its word: token row
  // 16 h + 8 (l / 32) + j' (+ 4 for the second read), channels wbase + 32 i + 16 (G' % 2) + 4 q'.
  const int L = lane & 15, jq = L >> 2, q = L & 3, g = (lane >> 4) & 1, kh = lane >> 5;
  const int wm = T.wave >> 1, wn = T.wave & 1;
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    const int wb32 = (o == 0 ? wm : wn) * 4;   // (wave's channel base) / 32
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 4 * (wb32 + (i ^ jq)) + 2 * g + (q >> 1);
      T.rd[o][i] = (uint32_t)(o * BM * kRowBytes) + (uint32_t)((8 * kh + jq) * kXRowBytes) +
                   (uint32_t)(pos * 16 + 8 * (q & 1));
    }
  }
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Fragment i (i < 4: A row block i, else B row block i - 4) of k half h from stage `st`.
__device__ __forceinline__ void kl_read_x(const char* smem, const TileX& T, int st, int h, int i,
                                          Frags& F) {
  const int o = i < 4 ? 0 : 1, blk = i & 3;
  const __attribute__((address_space(3))) char* base =
      (const __attribute__((address_space(3))) char*)smem + st * kStageBytes + T.rd[o][blk] +
      16 * h * kXRowBytes;
  const v4i16_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)base);
  const v4i16_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + 4 * kXRowBytes));
  // whole-vector casts and one shuffle (the halves stay in their registers)
  const half8_t f = __builtin_shufflevector(__builtin_bit_cast(half4_t, v0),
                                            __builtin_bit_cast(half4_t, v1), 0, 1, 2, 3, 4, 5,
                                            6, 7);
  if (o == 0)
    F.a[h][blk] = f;
  else
    F.b[h][blk] = f;
}

// Load slice idx in [0, 8) of step kt into stage `st` (even idx: A, odd: B; token rows
// 8 wave + 2 (idx / 2) .. + 1).
__device__ __forceinline__ void kl_issue_x(const TileX& T, int st, int kt, int idx) {
  const int j = idx >> 1;
  const uint32_t lds = T.lds0 + (uint32_t)(st * kStageBytes) + ((idx & 1) ? BM * kRowBytes : 0) +
                       (uint32_t)((T.wave * 8 + 2 * j) * kXRowBytes);
  const uint32_t so = T.soff + (uint32_t)(2 * j) * T.row_stride +
                      (uint32_t)(kt * BK) * T.row_stride;
  buffer_load16_lds_so((idx & 1) ? T.rb : T.ra, lds, T.voff[j & 1], so);
}

// kl_step with the X-operand reads and loads (no copies).
template <bool LO, bool HI, bool MORE, int VM>
__device__ __forceinline__ void kl_step_x(const char* smem, const TileX& T, int kt, Frags& F,
                                          floatx16 (&acc)[4][4]) {
  const int st = kt & 3;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[0][m >> 2], F.b[0][m & 3],
                                                                acc[m >> 2][m & 3], 0, 0, 0);
    if ((m & 1) == 0) kl_read_x(smem, T, st, 1, m >> 1, F);
    if (HI && (m & 3) == 1) kl_issue_x(T, (st + 3) & 3, kt + 3, 4 + (m >> 2));
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt(VM) & ~0x0F00);   // + lgkmcnt(0)
  __syncthreads();
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    acc[m >> 2][m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(F.a[1][m >> 2], F.b[1][m & 3],
                                                                acc[m >> 2][m & 3], 0, 0, 0);
    if (LO && (m & 3) == 0) kl_issue_x(T, st, kt + 4, m >> 2);
    if (MORE && (m & 1)) kl_read_x(smem, T, (st + 1) & 3, 0, m >> 1, F);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// kl_run on X operands (nk >= 4).
__device__ __forceinline__ void kl_run_x(const char* smem, const TileX& T, int nk,
                                         floatx16 (&acc)[4][4]) {
  Frags F;
#pragma unroll
  for (int p = 0; p < kStages; ++p)
#pragma unroll
    for (int idx = 0; idx < ((p < kStages - 1) ? 2 * kInstPerOp : kInstPerOp); ++idx)
      kl_issue_x(T, p, p, idx);
  __builtin_amdgcn_s_waitcnt(vmcnt(20));           // step 0 has landed
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) kl_read_x(smem, T, 0, 0, i, F);
  for (int kt = 0; kt < nk - 4; ++kt) kl_step_x<true, true, true, 16>(smem, T, kt, F, acc);
  kl_step_x<false, true, true, 16>(smem, T, nk - 4, F, acc);
  kl_step_x<false, false, true, 8>(smem, T, nk - 3, F, acc);
  kl_step_x<false, false, true, 0>(smem, T, nk - 2, F, acc);
  kl_step_x<false, false, false, 0>(smem, T, nk - 1, F, acc);
}

__device__ __forceinline__ void acc_zero(floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// Block b of a grid of G is dealt to XCD b % 8; returns the logical index that gives each XCD a
// contiguous range of the logical order.
__device__ __forceinline__ int xcd_logical(int b, int G) {
  const int per = G / 8, rem = G % 8, xcd = b % 8, loc = b / 8;
  return (xcd < rem) ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
}

}  // namespace kloop
}  // namespace awq
