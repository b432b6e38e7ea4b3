// fa_bwd_kernels.hpp -- device code of the attention backward on gfx950.
//   fa_bwd_pre     per (token, head) row: D = rowsum(O*dO) (step 4 of the
//                  PyPTO-Gym SK-16 article's per-tile math, section 3.1),
//                  the base-2 log-sum-exp of the forward's (m, l), a zeroed
//                  fp32 dQ accumulator row (single-pass form), and zeroed
//                  dQ/dK/dV rows outside every sequence. HBM bound.
//   fa_bwd_main    single-pass form, one workgroup per (kv tile, head,
//                  sequence): keeps the tile's K, V and its fp32 dK, dV
//                  accumulators in registers, streams the q tiles through LDS
//                  and runs the five GEMMs of steps 1, 3, 6, 7, 8 on bf16 MFMA
//                  with the softmax recompute and dS (steps 2, 5) on the VALU;
//                  dQ partial sums go to the fp32 accumulator with global
//                  atomics.
//   fa_bwd_dq_cast single-pass form: dQ = bf16(scale * accumulator). HBM bound.
//   fa_bwd_dkdv    recompute form, kv-outer: steps 1-3 and 5-7 with two
//                  waves per SIMD; dK, dV written once per kv tile.
//   fa_bwd_dq      recompute form, q-outer: recomputes S^T and dP^T and
//                  accumulates dQ (step 8) in registers; no atomics.
//   fa_fwd_fill,   the forward that produces O, m, l (the statistics step 2
//   fa_fwd         reads), for callers without one of their own.
// The recompute kernels and the forward also take grouped K/V heads and a
// sliding window (each query sees keys (i - w, i]).
#pragma once
#include <type_traits>

#include "cdna4.hpp"

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;

// First row and valid length of sequence b (layout in include/fa_bwd.h).
__device__ __forceinline__ void seq_of(const int* cu, int b, int padded, int max_seqlen, int64_t& start,
                                       int& len) {
  const int c0 = cu[b], c1 = cu[b + 1];
  len = c1 - c0;
  start = padded ? (int64_t)b * max_seqlen : (int64_t)c0;
}

// Does row t belong to some sequence?
__device__ __forceinline__ bool row_in_sequence(int64_t t, const int* cu, int batch, int padded, int max_seqlen) {
  if (padded) {
    const int64_t b = t / max_seqlen;
    if (b >= batch) return false;
    return (t - b * max_seqlen) < (int64_t)(cu[b + 1] - cu[b]);
  }
  return t >= cu[0] && t < cu[batch];
}

// ------------------------------------------------------------------ stage 1: row statistics

struct PreArgs {
  const bf16* o;
  const bf16* dout;
  const float* m;  // row max, or the log-sum-exp when l is null
  const float* l;  // row sum, or null
  const int* cu_q;
  const int* cu_kv;
  float* lse2;    // [H][total_q]: m*log2(e) + log2(l)
  float* dvec;    // [H][total_q]: rowsum(O*dO)
  float* dq_acc;  // [H][total_q][D], zeroed when not null
  bf16* dq;       // when not null: rows outside every sequence are zeroed
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded;  // query heads, K/V heads
};

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre(PreArgs a) {
  constexpr int TPR = D / 8;      // threads per (token, head) row, 8 elements each
  constexpr int RPB = 256 / TPR;  // rows per block
  const int sub = threadIdx.x % TPR;
  const int64_t pair = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;  // = t * H + h
  const int64_t t = pair / a.H;
  const int h = (int)(pair - t * a.H);
  const int64_t off = pair * D + sub * 8;
  if (t < a.total_q) {
    const bf16x8 ov = *(const bf16x8*)(a.o + off);
    const bf16x8 gv = *(const bf16x8*)(a.dout + off);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += from_bf16(ov[e]) * from_bf16(gv[e]);
#pragma unroll
    for (int s = TPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
    if (a.dq_acc) {
      float* accrow = a.dq_acc + ((int64_t)h * a.total_q + t) * D + sub * 8;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)accrow = z;
      *(f32x4*)(accrow + 4) = z;
    }
    if (a.dq && !row_in_sequence(t, a.cu_q, a.batch, a.padded, a.max_seqlen_q)) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      *(u32x4*)(a.dq + off) = z;
    }
    if (sub == 0) {
      const int64_t sidx = (int64_t)h * a.total_q + t;
      a.dvec[sidx] = acc;
      // (m, l) from the forward, or (when l is null) m holds the log-sum-exp m + ln(l) itself
      a.lse2[sidx] = a.l ? a.m[pair] * kLog2e + __log2f(a.l[pair]) : a.m[pair] * kLog2e;
    }
  }
  if (h < a.Hk && t < a.total_kv && !row_in_sequence(t, a.cu_kv, a.batch, a.padded, a.max_seqlen_kv)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int64_t koff = (t * a.Hk + h) * D + sub * 8;
    *(u32x4*)(a.dk + koff) = z;
    *(u32x4*)(a.dv + koff) = z;
  }
}

// ------------------------------------------------------------------ stage 2: single-pass main kernel

struct MainArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse2;
  const float* dvec;
  const int* cu_q;
  const int* cu_kv;
  float* dq_acc;  // fp32 [H][total_q][D] accumulator (single-pass form)
  bf16* dq;       // bf16 output (recompute form)
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded, causal;  // query heads, K/V heads (H % Hk == 0)
  int window;        // > 0: each query sees only its left local window of keys (i - window, i]
  float scale_log2;  // scale * log2(e)
  float scale;
};

template <int D>
struct MainCfg {
  static constexpr int BN = 128;                 // kv rows per workgroup (32 per wave)
  static constexpr int BM = 64;                  // q rows per step
  static constexpr int NW = 4;                   // waves
  static constexpr int KSD = D / 16;             // MFMA k-steps over the head dim
  static constexpr int NTD = D / 32;             // 32-wide output tiles over the head dim
  static constexpr int TPW = D / 64;             // dQ output tiles per wave
  static constexpr int QS = D + 8;               // row stride (elements) of the Q, dO and K tiles
  static constexpr int SS = BM + 8;              // row stride (elements) of dS^T
  static constexpr int CPR = QS / 8;             // 16-byte chunks per padded row
  static constexpr int TILE = BM * QS;           // elements of one Q or dO buffer
  static constexpr int TILE_BYTES = TILE * 2;
  static constexpr int NDMA = TILE_BYTES / 1024; // 1 KB LDS-DMA transfers per tile
  static constexpr int OFF_K = 0;                          // K tile [BN][QS]
  static constexpr int OFF_Q = OFF_K + BN * QS * 2;        // Q [2][BM][QS]
  static constexpr int OFF_DO = OFF_Q + 2 * TILE_BYTES;    // dO [2][BM][QS]
  static constexpr int OFF_DS = OFF_DO + 2 * TILE_BYTES;   // dS^T [BN][SS]
  static constexpr int OFF_ST = OFF_DS + BN * SS * 2;      // [2 buffers][lse2, D][BM] fp32
  static constexpr int LDS_BYTES = OFF_ST + 4 * BM * 4;
  static_assert(TILE_BYTES % 1024 == 0, "a tile is a whole number of 1 KB transfers");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Row of a 32-row M-tile (Q, dO) that MFMA row m reads, and kv row of the 128-row tile that
// k-index k of the dQ GEMM reads. With rows padded by 16 bytes, this interleave makes the
// 16-byte operand reads (16 consecutive m) and the 4-row transpose reads (m = 4u..4u+3)
// touch distinct LDS banks.
__device__ __forceinline__ constexpr int tile_row(int m) { return ((m >> 2) & 3) + 4 * (m & 3) + 16 * (m >> 4); }

constexpr int kRsrcWord3 = 0x00020000;

// Buffer resource over [base, base + bytes): loads past the end return 0 and atomics past
// the end are dropped (raw buffer, stride 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Rows [start, start + len) of a sequence, clamped to the rows that exist, so that
// every later row check is a single comparison against the length.
__device__ __forceinline__ int clamp_len(int64_t start, int len, int64_t total) {
  if (start < 0 || start >= total || len <= 0) return 0;
  return (int)((int64_t)len < total - start ? (int64_t)len : total - start);
}

__device__ __forceinline__ int imin(int x, int y) { return x < y ? x : y; }
__device__ __forceinline__ int imax(int x, int y) { return x > y ? x : y; }

// WITH_DQ: the single-pass form that also forms the dQ partial of every (q tile, kv tile)
// pair and adds it to the fp32 accumulator with atomics; without it the kernel produces dK
// and dV only and dQ comes from fa_bwd_dq.
template <int D, bool CAUSAL, bool WITH_DQ>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fa_bwd_main(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  using C = MainCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, QS = C::QS, SS = C::SS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  bf16* s_k = (bf16*)(smem + C::OFF_K);
  bf16* s_q = (bf16*)(smem + C::OFF_Q);
  bf16* s_do = (bf16*)(smem + C::OFF_DO);
  bf16* s_dst = (bf16*)(smem + C::OFF_DS);
  float* s_st = (float*)(smem + C::OFF_ST);

  const int HB = a.H * a.batch;
  const int tile = blockIdx.x / HB;  // heavy (low) kv tiles of every head dispatch first
  const int hb = blockIdx.x - tile * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int kv0 = tile * BN;
  if (kv0 >= Lk) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;  // elements between consecutive tokens
  const int rsb = (int)(rs * 2);        // bytes between consecutive tokens
  const bf16* kb = a.k + (kv_start + kv0) * rs + (int64_t)h * D;
  const bf16* vb = a.v + (kv_start + kv0) * rs + (int64_t)h * D;
  const bf16* qb = a.q + q_start * rs + (int64_t)h * D;
  const bf16* db = a.dout + q_start * rs + (int64_t)h * D;
  const float* lse_b = a.lse2 + (int64_t)h * a.total_q + q_start;
  const float* dd_b = a.dvec + (int64_t)h * a.total_q + q_start;
  float* dq_b = a.dq_acc + ((int64_t)h * a.total_q + q_start) * D;

  // ---- K tile -> LDS (kept for the dQ GEMM); K, V B-operand fragments of S and dP -> registers
  const int kv_rows = imin(Lk - kv0, BN);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (int64_t)kv_rows * rsb);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (int64_t)kv_rows * rsb);
  if constexpr (WITH_DQ) {
    for (int ch = tid; ch < BN * D / 8; ch += 256) {
      const int r = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(u32x4*)(s_k + r * QS + col) = buf_load16(rk, r * rsb + col * 2);
    }
  }
  bf16x8 kf[C::KSD], vf[C::KSD];
#pragma unroll
  for (int ks = 0; ks < C::KSD; ++ks) {
    const int off = (32 * w + c) * rsb + (16 * ks + 8 * hh) * 2;
    kf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  {  // zero both Q and dO buffers once: rows past the sequence then hold zeros or earlier valid rows
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < 4 * C::TILE_BYTES; o += 256 * 16) *(u32x4*)(smem + C::OFF_Q + o) = z;
  }
  __syncthreads();  // zero fill and K tile written before any LDS-DMA lands

  f32x16 accK[C::NTD], accV[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
    accK[nt] = f32x16{};
    accV[nt] = f32x16{};
  }

  const int n_qt = (Lq + BM - 1) / BM;
  int qt = CAUSAL ? kv0 / BM : 0;
  const int ntq = (w * C::TPW) >> 1;  // this wave's 32-wide feature slice of dQ
  const int jcol = kv0 + 32 * w + c;  // this lane's key row (sequence-local) in S and dP

  // LDS-DMA: transfer j lands lane L at tile byte 1024 j + 16 L = padded row (64 j + L) / CPR,
  // chunk (64 j + L) % CPR; the pad chunk re-reads chunk 0 of its row (never used).
  constexpr int NJ = (C::NDMA + C::NW - 1) / C::NW;
  int dma_off[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int p16 = 64 * (w + C::NW * jj) + lane;
    const int r = p16 / C::CPR, ch = p16 % C::CPR;
    dma_off[jj] = r * rsb + (ch < D / 8 ? ch : 0) * 16;
  }
  auto issue_tile = [&](int t, int bi) {
    const int i0 = t * BM;
    const int64_t bytes = (int64_t)imin(Lq - i0, BM) * rsb;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb + (int64_t)i0 * rs, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(db + (int64_t)i0 * rs, bytes);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(smem + C::OFF_Q + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rd, (__attribute__((address_space(3))) void*)(smem + C::OFF_DO + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
      }
    }
  };
  // row statistics of q tile t in MFMA row order: threads 0..63 lse2, 64..127 D. Rows past the
  // sequence get lse2 = +inf, so their P (and dS) is exactly 0 without a mask.
  auto load_stats = [&](int t) -> float {
    const int mi = tid & (BM - 1);
    const int r = t * BM + 32 * (mi >> 5) + tile_row(mi & 31);
    if (tid >= 2 * BM) return 0.f;
    if (r >= Lq) return tid < BM ? __builtin_inff() : 0.f;
    return (tid < BM ? lse_b : dd_b)[r];
  };
  auto store_stats = [&](int bi, float v) {
    if (tid < 2 * BM) s_st[bi * 2 * BM + tid] = v;
  };

  // one q tile: steps 1-7 of the per-tile math for this wave's 32 keys. Keys past the sequence
  // need no mask: their K rows are zero in LDS (no dQ contribution) and their dK/dV rows are
  // never written. Only the causal predicate is applied.
  auto tile_step = [&](int bi, int i0) {
    const bf16* sq = s_q + bi * C::TILE;
    const bf16* sd = s_do + bi * C::TILE;
    const float* st = s_st + bi * 2 * BM;
    const int jrel = jcol - i0;  // causal: key j is visible from tile row r iff jrel <= r
    const int arow = tile_row(c) * QS + 8 * hh;
    const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);
    // steps 1 and 3 for M-tile mt: S = Q K^T, dP = dO V^T  ([q 32] x [kv 32] per wave)
    auto sdp = [&](int mt, f32x16& s, f32x16& dp) {
      s = f32x16{};
      dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::KSD; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(sq + arow + 32 * mt * QS + 16 * ks);
        const bf16x8 da = *(const bf16x8*)(sd + arow + 32 * mt * QS + 16 * ks);
        s = mfma32x32x16(qa, kf[ks], s);
        dp = mfma32x32x16(da, vf[ks], dp);
      }
    };
    // steps 2 and 5 for M-tile mt: P = exp2(S*scale*log2e - lse2), dS = P (dP - D), both to bf16
    auto softmax_ds = [&](int mt, const f32x16& s, const f32x16& dp, bf16x8 (&pk)[2], bf16x8 (&dsk)[2]) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int mrow = 32 * mt + 8 * a4 + 4 * hh;  // MFMA row of bb = 0
        const f32x4 lse = *(const f32x4*)(st + mrow);
        const f32x4 dd = *(const f32x4*)(st + BM + mrow);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int j = 4 * a4 + bb;
          float p = fast_exp2(s[j] * a.scale_log2 - lse[bb]);
          if constexpr (CAUSAL) p = (jrel <= 32 * mt + tile_row(8 * a4 + 4 * hh + bb)) ? p : 0.f;
          const float ds = p * (dp[j] - dd[bb]);
          pk[j >> 3][j & 7] = to_bf16(p);
          dsk[j >> 3][j & 7] = to_bf16(ds);
        }
      }
    };
    // steps 7 and 6 for M-tile mt: dV += P^T dO, dK += dS^T Q (scale applied at write-back). The
    // k-index e of the A operand is MFMA row 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4;
    // the transpose reads fetch the matching tile rows.
    auto dvdk = [&](int mt, const bf16x8 (&pk)[2], const bf16x8 (&dsk)[2]) {
#pragma unroll
      for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int o = brow + (32 * mt + 16 * s2) * QS + 32 * nt;
          const bf16x8 bdo = concat(lds_read_tr4(sd + o), lds_read_tr4(sd + o + 2 * QS));
          const bf16x8 bq = concat(lds_read_tr4(sq + o), lds_read_tr4(sq + o + 2 * QS));
          accV[nt] = mfma32x32x16(pk[s2], bdo, accV[nt]);
          accK[nt] = mfma32x32x16(dsk[s2], bq, accK[nt]);
        }
      }
    };
    // Software pipeline over the two M-tiles: the softmax of one M-tile runs on the VALU while
    // the matrix cores work on the other's GEMMs.
    f32x16 s0, dp0, s1, dp1;
    bf16x8 pk0[2], dsk0[2], pk1[2], dsk1[2];
    sdp(0, s0, dp0);
    sdp(1, s1, dp1);
    softmax_ds(0, s0, dp0, pk0, dsk0);
    dvdk(0, pk0, dsk0);
    softmax_ds(1, s1, dp1, pk1, dsk1);
    dvdk(1, pk1, dsk1);
    // interleave: [S/dP 0] [S/dP 1 | softmax 0] [dV/dK 0 | softmax 1] [dV/dK 1]
#pragma unroll
    for (int i = 0; i < C::KSD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 DS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
    }
#pragma unroll
    for (int i = 0; i < C::KSD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 112 / C::KSD, 0);  // softmax VALU
    }
#pragma unroll
    for (int i = 0; i < 2 * C::NTD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 112 / (2 * C::NTD), 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * C::NTD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    // dS^T to LDS (for the dQ GEMM): row = this lane's key, 4 consecutive MFMA rows per store
    if constexpr (WITH_DQ) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const bf16x8 src = (mt == 0 ? dsk0 : dsk1)[a4 >> 1];
          const int o4 = 4 * (a4 & 1);
          const bf16x4 v4 = {src[o4], src[o4 + 1], src[o4 + 2], src[o4 + 3]};
          *(bf16x4*)(s_dst + (32 * w + c) * SS + 32 * mt + 8 * a4 + 4 * hh) = v4;
        }
      }
    }
  };

  int buf = 0;
  if (qt < n_qt) {
    issue_tile(qt, 0);
    store_stats(0, load_stats(qt));
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  for (; qt < n_qt; ++qt, buf ^= 1) {
    const bool has_next = qt + 1 < n_qt;
    float st_next = 0.f;
    if (has_next) {
      issue_tile(qt + 1, buf ^ 1);
      st_next = load_stats(qt + 1);
    }
    const int i0 = qt * BM;
    tile_step(buf, i0);
    if constexpr (!WITH_DQ) {
      if (has_next) store_stats(buf ^ 1, st_next);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next tile's LDS-DMA has landed
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      continue;
    }
    __syncthreads();  // dS^T complete
    if (has_next) store_stats(buf ^ 1, st_next);

    // step 8: dQ partial = dS K over this tile's 128 keys, added to the fp32 accumulator.
    // k-index 16 ks + 8 hh + 4 half + e reads kv row 16 ks + 2 hh + half + 4 e.
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(dq_b + (int64_t)i0 * D, (int64_t)imin(Lq - i0, BM) * D * 4);
    const int krow = 2 * hh + 4 * (gi >> 2);
    const int tcol = 16 * (g & 1) + 4 * (gi & 3);
#pragma unroll
    for (int tt = 0; tt < C::TPW; ++tt) {
      const int mtq = (w * C::TPW + tt) & 1;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const int ra = (16 * ks + krow) * SS + 32 * mtq + tcol;
        const int rb = (16 * ks + krow) * QS + 32 * ntq + tcol;
        const bf16x8 af = concat(lds_read_tr4(s_dst + ra), lds_read_tr4(s_dst + ra + SS));
        const bf16x8 bk = concat(lds_read_tr4(s_k + rb), lds_read_tr4(s_k + rb + QS));
        acc = mfma32x32x16(af, bk, acc);
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int row = 32 * mtq + tile_row(8 * a4 + 4 * hh + bb);
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[4 * a4 + bb], rq, (row * D + 32 * ntq + c) * 4, 0, 0);
        }
      }
    }
    // the next tile's LDS-DMA (issued before this tile's atomics) must land before the barrier
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(16 * C::TPW));
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // write-back: dK = scale * accK, dV = accV, bf16, rows of this wave's keys
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = kv0 + 32 * w + 8 * a4 + 4 * hh + bb;
        if (r < Lk) {
          const int64_t o = (kv_start + r) * rs + (int64_t)h * D + 32 * nt + c;
          a.dk[o] = to_bf16(accK[nt][4 * a4 + bb] * a.scale);
          a.dv[o] = to_bf16(accV[nt][4 * a4 + bb]);
        }
      }
    }
  }
#endif
}


// ------------------------------------------------------------------ stage 2a: dK and dV by recompute

template <int D>
struct DkdvCfg {
  static constexpr int BN = 128;                 // kv rows per workgroup: 4 row groups of 32
  static constexpr int BM = 64;                  // q rows per step: 2 M-tiles of 32
  static constexpr int NW = 8;                   // waves: 4 row groups x 2 M-tiles
  static constexpr int NT = 64 * NW;
  static constexpr int KSD = D / 16;
  static constexpr int NTD = D / 32;
  static constexpr int QS = D + 8;               // padded row stride of every LDS tile
  static constexpr int CPR = QS / 8;
  static constexpr int TILE = BM * QS;
  static constexpr int TILE_BYTES = TILE * 2;
  static constexpr int NDMA = TILE_BYTES / 1024;
  static constexpr int KV_BYTES = BN * QS * 2;   // the K (or V) tile of the workgroup
  static constexpr int NDMA_KV = KV_BYTES / 1024;
  static constexpr int OFF_K = 0;                             // K [BN][QS]
  static constexpr int OFF_V = OFF_K + KV_BYTES;              // V [BN][QS]
  static constexpr int OFF_Q = OFF_V + KV_BYTES;              // Q [2][BM][QS]
  static constexpr int OFF_DO = OFF_Q + 2 * TILE_BYTES;       // dO [2][BM][QS]
  static constexpr int OFF_ST = OFF_DO + 2 * TILE_BYTES;      // [2 buffers][lse2, D][BM] fp32
  static constexpr int LDS_BYTES = OFF_ST + 4 * BM * 4;
  static constexpr int PART_BYTES = NTD * 16 * 4 * 64;        // one wave's partial dK or dV tile
  static_assert(TILE_BYTES % 1024 == 0 && KV_BYTES % 1024 == 0, "tiles are whole 1 KB transfers");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget (one 8-wave workgroup per CU)");
  static_assert(NW * PART_BYTES <= OFF_ST, "the end-of-kernel exchange of partial sums fits in the tiles");
};

// dK and dV of one (kv tile, K/V head, sequence). Eight waves: row group r = w % 4 owns kv rows
// 32 r .. 32 r + 31, and the two waves of a group each take one 32-row M-tile mt = w / 4 of every
// 64-row q step. Each wave forms S = Q K^T, dP = dO V^T, P and dS for its M-tile (steps 1-5) and
// accumulates its partial dV += P^T dO and dK += dS^T Q over its M-tile's rows (steps 7, 6), so
// the waves of a step never wait for each other; K and V are read from an LDS tile loaded once,
// which leaves registers for both accumulators. After the last step the two waves of a group
// combine their partial sums through LDS (the M-tile 0 wave finishes dV, the other dK).
template <int D, bool CAUSAL, bool WINDOW>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dkdv(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DkdvCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, QS = C::QS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
  const bf16* s_k = (const bf16*)(smem + C::OFF_K);
  const bf16* s_v = (const bf16*)(smem + C::OFF_V);
  bf16* s_q = (bf16*)(smem + C::OFF_Q);
  bf16* s_do = (bf16*)(smem + C::OFF_DO);
  float* s_st = (float*)(smem + C::OFF_ST);

  const int HB = a.Hk * a.batch;
  const int tile = blockIdx.x / HB;  // heavy (low) kv tiles of every head dispatch first
  const int hb = blockIdx.x - tile * HB;
  const int b = hb / a.Hk, hk = hb - (hb / a.Hk) * a.Hk;  // sequence, K/V head
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int kv0 = tile * BN;
  if (kv0 >= Lk) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int grp = w & 3, mt = w >> 2;  // kv row group; M-tile
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;    // row stride of Q, dO
  const int rsb = (int)(rs * 2);
  const int64_t rsk = (int64_t)a.Hk * D;  // row stride of K, V, dK, dV
  const int rskb = (int)(rsk * 2);
  const int G = a.H / a.Hk;               // query heads sharing this K/V head: hk * G .. hk * G + G - 1

  {  // zero the tiles once: rows past the sequences then hold zeros or earlier valid rows
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::OFF_ST; o += C::NT * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  // the q steps: for each query head of the group, the q tiles that can see these keys (causal: from
  // the tile of the first key on); step st is q tile qt0 + st % nq of query head hk * G + st / nq
  const int n_qt = (Lq + BM - 1) / BM;
  const int qt0 = CAUSAL ? kv0 / BM : 0;
  // window: the last query that sees a key of this tile is kv0 + BN - 2 + window
  const int qt_end = WINDOW ? imin(n_qt, (kv0 + BN - 2 + a.window) / BM + 1) : n_qt;
  const int nq = qt_end > qt0 ? qt_end - qt0 : 0;
  const int n_steps = G * nq;
  auto step_head = [&](int st) { return hk * G + st / nq; };
  auto step_tile = [&](int st) { return qt0 + st % nq; };
  const int jcol = kv0 + 32 * grp + c;  // this lane's key row (sequence-local)

  // 1 KB LDS-DMA transfers of padded rows: transfer j, lane -> row p16 / CPR, 16-byte chunk p16 % CPR
  auto dma_row_off = [&](int j, int row_bytes) {
    const int p16 = 64 * j + lane;
    const int r = p16 / C::CPR, ch = p16 % C::CPR;
    return r * row_bytes + (ch < D / 8 ? ch : 0) * 16;
  };
  {  // the K and V tiles, once
    const int kv_rows = imin(Lk - kv0, BN);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (kv_start + kv0) * rsk + (int64_t)hk * D, (int64_t)kv_rows * rskb);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (kv_start + kv0) * rsk + (int64_t)hk * D, (int64_t)kv_rows * rskb);
    for (int j = w; j < C::NDMA_KV; j += C::NW) {
      const int off = dma_row_off(j, rskb);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(smem + C::OFF_K + 1024 * j),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(smem + C::OFF_V + 1024 * j),
                                               16, off, 0, 0, 0);
    }
  }
  constexpr int NJ = (C::NDMA + C::NW - 1) / C::NW;
  int dma_off[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) dma_off[jj] = dma_row_off(w + C::NW * jj, rsb);
  auto issue_tile = [&](int st, int bi) {
    const int i0 = step_tile(st) * BM;
    const int64_t hoff = (q_start + i0) * rs + (int64_t)step_head(st) * D;
    const int64_t bytes = (int64_t)imin(Lq - i0, BM) * rsb;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + hoff, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + hoff, bytes);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rq, (__attribute__((address_space(3))) void*)(smem + C::OFF_Q + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rd, (__attribute__((address_space(3))) void*)(smem + C::OFF_DO + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
      }
    }
  };
  // row statistics of a q step in MFMA row order: threads 0..63 lse2, 64..127 D; rows past the
  // sequence get lse2 = +inf, so their P (and dS) is exactly 0 without a mask
  auto load_stats = [&](int st) -> float {
    const int mi = tid & (BM - 1);
    const int r = step_tile(st) * BM + 32 * (mi >> 5) + tile_row(mi & 31);
    if (tid >= 2 * BM) return 0.f;
    if (r >= Lq) return tid < BM ? __builtin_inff() : 0.f;
    const int64_t sidx = (int64_t)step_head(st) * a.total_q + q_start + r;
    return (tid < BM ? a.lse2 : a.dvec)[sidx];
  };
  auto store_stats = [&](int bi, float v) {
    if (tid < 2 * BM) s_st[bi * 2 * BM + tid] = v;
  };

  f32x16 acc_v[C::NTD], acc_k[C::NTD];  // partial dV and dK / scale of rows 32 grp .. +31 over this M-tile
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
    acc_v[nt] = f32x16{};
    acc_k[nt] = f32x16{};
  }

  int buf = 0;
  if (n_steps > 0) {
    issue_tile(0, 0);
    store_stats(0, load_stats(0));
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  const int arow = (32 * mt + tile_row(c)) * QS + 8 * hh;  // A rows: this M-tile's q rows
  const int krow = (32 * grp + c) * QS + 8 * hh;            // B columns: this group's keys
  const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3) + 32 * mt * QS;
  for (int sp = 0; sp < n_steps; ++sp, buf ^= 1) {
    const bool has_next = sp + 1 < n_steps;
    float st_next = 0.f;
    if (has_next) {
      issue_tile(sp + 1, buf ^ 1);
      st_next = load_stats(sp + 1);
    }
    const int i0 = step_tile(sp) * BM;
    const bf16* sq = s_q + buf * C::TILE;
    const bf16* sd = s_do + buf * C::TILE;
    const float* st = s_st + buf * 2 * BM + 32 * mt;
    // steps 1 and 3 for this wave's M-tile: S = Q K^T, dP = dO V^T  ([q 32] x [kv 32]); operands
    // are read PF k-steps ahead into distinct registers, one scheduling fence per k-step
    f32x16 s = f32x16{}, dp = f32x16{};
    {
      constexpr int PF = 2;
      bf16x8 qa[C::KSD], da[C::KSD], kb[C::KSD], vb[C::KSD];
      auto ld = [&](int ks) {
        qa[ks] = *(const bf16x8*)(sq + arow + 16 * ks);
        da[ks] = *(const bf16x8*)(sd + arow + 16 * ks);
        kb[ks] = *(const bf16x8*)(s_k + krow + 16 * ks);
        vb[ks] = *(const bf16x8*)(s_v + krow + 16 * ks);
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) ld(ks);
#pragma unroll
      for (int ks = 0; ks < C::KSD; ++ks) {
        if (ks + PF < C::KSD) ld(ks + PF);
        s = mfma32x32x16(qa[ks], kb[ks], s);
        dp = mfma32x32x16(da[ks], vb[ks], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // steps 2 and 5: P = exp2(S*scale*log2e - lse2) (causal: 0 where key > query), dS = P (dP - D)
    const int jrel = jcol - i0 - 32 * mt;  // key j visible from M-tile row r iff jrel <= r
    bf16x8 pk[2], dsk[2];
    auto softmax = [&](auto masked) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 lse = *(const f32x4*)(st + 8 * a4 + 4 * hh);
        const f32x4 dd = *(const f32x4*)(st + BM + 8 * a4 + 4 * hh);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int j = 4 * a4 + bb;
          float p = fast_exp2(s[j] * a.scale_log2 - lse[bb]);
          if constexpr (decltype(masked)::value) {
            const int r = tile_row(8 * a4 + 4 * hh + bb);
            if constexpr (WINDOW)  // key j visible from query i iff i - window < j <= i
              p = (jrel <= r && r - jrel < a.window) ? p : 0.f;
            else
              p = (jrel <= r) ? p : 0.f;
          }
          pk[j >> 3][j & 7] = to_bf16(p);
          dsk[j >> 3][j & 7] = to_bf16(p * (dp[j] - dd[bb]));
        }
      }
    };
    // every key of the group visible from every query of the M-tile: no element mask (wave-uniform)
    const int kmin = kv0 + 32 * grp, qmin = i0 + 32 * mt;
    const bool full = !CAUSAL || (kmin + 31 <= qmin && (!WINDOW || qmin + 31 - a.window < kmin));
    if (full)
      softmax(std::false_type{});
    else
      softmax(std::true_type{});
    // steps 7 and 6 over this M-tile: dV += P^T dO, dK += dS^T Q. k-step s2: its k-index e is MFMA
    // row 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4; the transpose reads fetch those rows.
    // B operands are read PF MFMAs ahead; the dV and dK MFMAs alternate (independent chains).
    {
      constexpr int NB = 2 * C::NTD, PF = 2;
      bf16x8 bd[NB], bq[NB];
      auto ld = [&](int i) {
        const int s2 = i / C::NTD, nt = i % C::NTD;
        const int o = brow + 16 * s2 * QS + 32 * nt;
        bd[i] = concat(lds_read_tr4(sd + o), lds_read_tr4(sd + o + 2 * QS));
        bq[i] = concat(lds_read_tr4(sq + o), lds_read_tr4(sq + o + 2 * QS));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) ld(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i + PF < NB) ld(i + PF);
        const int s2 = i / C::NTD, nt = i % C::NTD;
        acc_v[nt] = mfma32x32x16(pk[s2], bd[i], acc_v[nt]);
        acc_k[nt] = mfma32x32x16(dsk[s2], bq[i], acc_k[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (has_next) store_stats(buf ^ 1, st_next);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next tile's LDS-DMA has landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // combine the two M-tiles' partial sums: the M-tile 0 wave keeps dV and takes the partner's dV,
  // the M-tile 1 wave keeps dK and takes the partner's dK; each writes the half its partner needs
  {
    f32x16* part = (f32x16*)(smem) + (size_t)w * C::NTD * 64 + lane;  // [wave][nt][lane]
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) part[nt * 64] = mt == 0 ? acc_k[nt] : acc_v[nt];
  }
  __syncthreads();
  {
    const f32x16* other = (const f32x16*)(smem) + (size_t)(w ^ 4) * C::NTD * 64 + lane;
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
      if (mt == 0) acc_v[nt] += other[nt * 64];
      else acc_k[nt] += other[nt * 64];
    }
  }
  // write-back: M-tile 0 wave dV, M-tile 1 wave dK = scale * acc, bf16, rows 32 grp .. 32 grp + 31
  bf16* out = mt == 0 ? a.dv : a.dk;
  const float osc = mt == 0 ? 1.f : a.scale;
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
    const f32x16 res = mt == 0 ? acc_v[nt] : acc_k[nt];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = kv0 + 32 * grp + 8 * a4 + 4 * hh + bb;
        if (r < Lk) out[(kv_start + r) * rsk + (int64_t)hk * D + 32 * nt + c] = to_bf16(res[4 * a4 + bb] * osc);
      }
    }
  }
#endif
}

// ------------------------------------------------------------------ stage 2b: dQ by recompute


template <int D>
struct DqCfg {
  static constexpr int BQ = 128;                 // q rows per workgroup (32 per wave)
  static constexpr int BK = 64;                  // kv rows per step
  static constexpr int NW = 4;
  static constexpr int KSD = D / 16;
  static constexpr int NTD = D / 32;
  static constexpr int QS = D + 8;               // padded row stride of the K and V tiles
  static constexpr int CPR = QS / 8;
  static constexpr int TILE = BK * QS;
  static constexpr int TILE_BYTES = TILE * 2;
  static constexpr int NDMA = TILE_BYTES / 1024;
  static constexpr int OFF_K = 0;                          // K [2][BK][QS]
  static constexpr int OFF_V = OFF_K + 2 * TILE_BYTES;     // V [2][BK][QS]
  static constexpr int LDS_BYTES = OFF_V + 2 * TILE_BYTES;
  static_assert(TILE_BYTES % 1024 == 0, "a tile is a whole number of 1 KB transfers");
};

// dQ of one (q tile, head, sequence): loops over the kv tiles, recomputes S^T = K Q^T and
// dP^T = V dO^T with the forward's statistics (steps 1-5 of the per-tile math), and
// accumulates dQ^T = K^T dS^T (step 8) in registers; dQ is written once, in bf16.
template <int D, bool CAUSAL, bool WINDOW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqCfg<D>;
  constexpr int BQ = C::BQ, BK = C::BK, QS = C::QS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int HB = a.H * a.batch;
  const int tr = blockIdx.x / HB;
  const int hb = blockIdx.x - tr * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  // causal: the q tiles with the most keys (the last ones) dispatch first
  const int n_qt_max = (a.max_seqlen_q + BQ - 1) / BQ;
  const int qtile = CAUSAL ? n_qt_max - 1 - tr : tr;
  const int i0 = qtile * BQ;
  if (i0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;    // row stride of the query-side tensors
  const int rsb = (int)(rs * 2);
  const int64_t rsk = (int64_t)a.Hk * D;  // row stride of K, V
  const int rskb = (int)(rsk * 2);
  const int hk = h / (a.H / a.Hk);        // the K/V head this query head reads
  const bf16* kb = a.k + kv_start * rsk + (int64_t)hk * D;
  const bf16* vb = a.v + kv_start * rsk + (int64_t)hk * D;
  const bf16* qb = a.q + (q_start + i0) * rs + (int64_t)h * D;
  const bf16* db = a.dout + (q_start + i0) * rs + (int64_t)h * D;
  const int qi = i0 + 32 * w + c;  // this lane's query row (sequence-local) in S^T, dP^T and dQ^T

  // Q, dO as B operands of S^T = K Q^T and dP^T = V dO^T: row qi, features 16 ks + 8 hh ..+7
  const int q_rows = imin(Lq - i0, BQ);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)q_rows * rsb);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(db, (int64_t)q_rows * rsb);
  bf16x8 qf[C::KSD], df[C::KSD];
#pragma unroll
  for (int ks = 0; ks < C::KSD; ++ks) {
    const int off = (32 * w + c) * rsb + (16 * ks + 8 * hh) * 2;
    qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[ks] = __builtin_bit_cast(bf16x8, buf_load16(rd, off));
  }
  // rows past the sequence: lse2 = +inf makes P (and dS) exactly 0
  const float lse = qi < Lq ? a.lse2[(int64_t)h * a.total_q + q_start + qi] : __builtin_inff();
  const float dd = qi < Lq ? a.dvec[(int64_t)h * a.total_q + q_start + qi] : 0.f;

  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);
  // window: the first query of the tile sees no key before i0 - window + 1
  const int t0 = WINDOW ? imax(0, i0 - a.window + 1) / BK : 0;

  {  // zero the K and V buffers once (rows past the sequence are masked, but must be finite)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::LDS_BYTES; o += 256 * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  constexpr int NJ = (C::NDMA + C::NW - 1) / C::NW;
  int dma_off[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int p16 = 64 * (w + C::NW * jj) + lane;
    const int r = p16 / C::CPR, ch = p16 % C::CPR;
    dma_off[jj] = r * rskb + (ch < D / 8 ? ch : 0) * 16;
  }
  auto issue_kv = [&](int t, int bi) {
    const int j0 = t * BK;
    const int64_t bytes = (int64_t)imin(Lk - j0, BK) * rskb;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (int64_t)j0 * rsk, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb + (int64_t)j0 * rsk, bytes);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(smem + C::OFF_K + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(smem + C::OFF_V + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
      }
    }
  };

  f32x16 acc[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) acc[nt] = f32x16{};

  int buf = 0;
  if (n_kt > t0) issue_kv(t0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  const int arow = tile_row(c) * QS + 8 * hh;
  const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);
  for (int t = t0; t < n_kt; ++t, buf ^= 1) {
    if (t + 1 < n_kt) issue_kv(t + 1, buf ^ 1);
    const bf16* sk = (const bf16*)(smem + C::OFF_K + buf * C::TILE_BYTES);
    const bf16* sv = (const bf16*)(smem + C::OFF_V + buf * C::TILE_BYTES);
    // steps 1 and 3, transposed: S^T = K Q^T, dP^T = V dO^T  ([kv 64] x [q 32] per wave)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      dp[mt] = f32x16{};
    }
    {  // operands read PF k-steps ahead into distinct registers, one scheduling fence per k-step
      constexpr int PF = 2;
      bf16x8 ka[C::KSD][2], va[C::KSD][2];
      auto ld = [&](int ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          ka[ks][mt] = *(const bf16x8*)(sk + arow + 32 * mt * QS + 16 * ks);
          va[ks][mt] = *(const bf16x8*)(sv + arow + 32 * mt * QS + 16 * ks);
        }
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) ld(ks);
#pragma unroll
      for (int ks = 0; ks < C::KSD; ++ks) {
        if (ks + PF < C::KSD) ld(ks + PF);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          s[mt] = mfma32x32x16(ka[ks][mt], qf[ks], s[mt]);
          dp[mt] = mfma32x32x16(va[ks][mt], df[ks], dp[mt]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // steps 2 and 5: P = exp2(S*scale*log2e - lse2), dS = P (dP - D); key row j = t*BK + kv row.
    // Visible iff j < Lk and (causal) j <= qi: one bound per lane on the tile-local kv row.
    const int lim = CAUSAL ? imin(Lk - 1, qi) - t * BK : Lk - 1 - t * BK;
    const int lo = qi - a.window + 1 - t * BK;  // window: first visible tile-local key
    bf16x8 dsk[2][2];
    auto softmax = [&](auto masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int j = 4 * a4 + bb;
            float p = fast_exp2(s[mt][j] * a.scale_log2 - lse);
            if constexpr (decltype(masked)::value) {
              const int kr = 32 * mt + tile_row(8 * a4 + 4 * hh + bb);
              p = (kr <= lim && (!WINDOW || kr >= lo)) ? p : 0.f;
            }
            dsk[mt][j >> 3][j & 7] = to_bf16(p * (dp[mt][j] - dd));
          }
        }
      }
    };
    // every key of the tile visible from every row of this wave: no element mask (wave-uniform)
    const int qmin = i0 + 32 * w, kmax = t * BK + BK - 1;
    const bool full = kmax <= Lk - 1 && (!CAUSAL || kmax <= qmin) && (!WINDOW || qmin + 31 - a.window < t * BK);
    if (full)
      softmax(std::false_type{});
    else
      softmax(std::true_type{});
    // step 8, transposed: dQ^T += K^T dS^T. k-step ksi = 2 mt + s2: its k-index e is kv MFMA row
    // 16 s2 + 4 hh + e (e < 4) or 16 s2 + 8 + 4 hh + e - 4 of M-tile mt; the transpose reads fetch
    // those K rows. k-steps run outside the NTD independent accumulators; A operands are read PF
    // MFMAs ahead.
    {
      constexpr int NB = 4 * C::NTD, PF = 3;
      bf16x8 kt[NB];
      auto kt_load = [&](int i) {
        const int ksi = i / C::NTD, nt = i % C::NTD;
        const int o = brow + 16 * ksi * QS + 32 * nt;
        return concat(lds_read_tr4(sk + o), lds_read_tr4(sk + o + 2 * QS));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) kt[i] = kt_load(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i + PF < NB) kt[i + PF] = kt_load(i + PF);
        const int ksi = i / C::NTD, nt = i % C::NTD;
        acc[nt] = mfma32x32x16(kt[i], dsk[ksi >> 1][ksi & 1], acc[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next K/V tiles have landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // dQ = scale * (dQ^T)^T in bf16: this lane holds features 32 nt + 8 a4 + 4 hh + bb of row qi
  if (qi < Lq) {
    bf16* dst = a.dq + (q_start + qi) * rs + (int64_t)h * D + 4 * hh;
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const bf16x4 v4 = {to_bf16(acc[nt][4 * a4] * a.scale), to_bf16(acc[nt][4 * a4 + 1] * a.scale),
                           to_bf16(acc[nt][4 * a4 + 2] * a.scale), to_bf16(acc[nt][4 * a4 + 3] * a.scale)};
        *(bf16x4*)(dst + 32 * nt + 8 * a4) = v4;
      }
    }
  }
#endif
}

// ------------------------------------------------------------------ forward: O, m, l

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int* cu_q;
  const int* cu_kv;
  bf16* o;   // [total_q][H][D]
  float* m;  // [total_q][H]: row max of the scaled visible logits
  float* l;  // [total_q][H]: row sum of exp(scaled logit - m) over visible keys
  int64_t total_q, total_kv;
  int H, Hk, batch, max_seqlen_q, max_seqlen_kv, padded;  // query heads, K/V heads (H % Hk == 0)
  int window;        // > 0: each query sees only its left local window of keys (i - window, i]
  float scale_log2;  // scale * log2(e)
};

// Rows outside every sequence: O = 0, m = 0, l = 1 (finite values a backward never reads).
template <int D>
__global__ __launch_bounds__(256) void fa_fwd_fill(FwdArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const int64_t pair = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;  // = t * H + h
  const int64_t t = pair / a.H;
  if (t >= a.total_q || row_in_sequence(t, a.cu_q, a.batch, a.padded, a.max_seqlen_q)) return;
  const u32x4 z = {0u, 0u, 0u, 0u};
  *(u32x4*)(a.o + pair * D + sub * 8) = z;
  if (sub == 0) {
    a.m[pair] = 0.f;
    a.l[pair] = 1.f;
  }
}

// Forward of one (q tile, head, sequence), the producer of the backward's inputs: S^T = K Q^T on
// bf16 MFMA, softmax with a running row maximum (the forward that the per-tile backward math
// inverts: P = exp(S*scale - m) / l), O^T += V^T P^T in registers; O = O^T^T / l, m and l written
// once per row. Same tiling as the dQ kernel: Q in registers, K and V tiles of 64 keys streamed
// through LDS, each lane owns one query row (its MFMA column), so the running maximum, the row sum
// and the rescaling of its O row are per-lane values combined with the partner lane (lane ^ 32).
template <int D, bool CAUSAL, bool WINDOW>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_fwd(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqCfg<D>;
  constexpr int BQ = C::BQ, BK = C::BK, QS = C::QS;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int HB = a.H * a.batch;
  const int tr = blockIdx.x / HB;
  const int hb = blockIdx.x - tr * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int n_qt_max = (a.max_seqlen_q + BQ - 1) / BQ;
  const int qtile = CAUSAL ? n_qt_max - 1 - tr : tr;  // causal: q tiles with the most keys first
  const int i0 = qtile * BQ;
  if (i0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;    // row stride of the query-side tensors
  const int rsb = (int)(rs * 2);
  const int64_t rsk = (int64_t)a.Hk * D;  // row stride of K, V
  const int rskb = (int)(rsk * 2);
  const int hk = h / (a.H / a.Hk);        // the K/V head this query head reads
  const bf16* kb = a.k + kv_start * rsk + (int64_t)hk * D;
  const bf16* vb = a.v + kv_start * rsk + (int64_t)hk * D;
  const bf16* qb = a.q + (q_start + i0) * rs + (int64_t)h * D;
  const int qi = i0 + 32 * w + c;  // this lane's query row (sequence-local)

  const int q_rows = imin(Lq - i0, BQ);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (int64_t)q_rows * rsb);
  bf16x8 qf[C::KSD];
#pragma unroll
  for (int ks = 0; ks < C::KSD; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8, buf_load16(rq, (32 * w + c) * rsb + (16 * ks + 8 * hh) * 2));

  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);
  // window: the first query of the tile sees no key before i0 - window + 1
  const int t0 = WINDOW ? imax(0, i0 - a.window + 1) / BK : 0;

  {  // zero the K and V buffers once (keys past the sequence are masked, but must be finite)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::LDS_BYTES; o += 256 * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  constexpr int NJ = (C::NDMA + C::NW - 1) / C::NW;
  int dma_off[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int p16 = 64 * (w + C::NW * jj) + lane;
    const int r = p16 / C::CPR, ch = p16 % C::CPR;
    dma_off[jj] = r * rskb + (ch < D / 8 ? ch : 0) * 16;
  }
  auto issue_kv = [&](int t, int bi) {
    const int j0 = t * BK;
    const int64_t bytes = (int64_t)imin(Lk - j0, BK) * rskb;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (int64_t)j0 * rsk, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb + (int64_t)j0 * rsk, bytes);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(smem + C::OFF_K + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(smem + C::OFF_V + bi * C::TILE_BYTES + 1024 * j), 16,
            dma_off[jj], 0, 0, 0);
      }
    }
  };

  f32x16 acc[C::NTD];  // O^T of this lane's row: features 32 nt + 8 a4 + 4 hh + bb
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) acc[nt] = f32x16{};
  float mrun = -__builtin_inff();  // running max of S*scale*log2(e) over the keys seen
  float lrun = 0.f;                // this lane's part of sum exp2(S*scale*log2(e) - mrun)

  int buf = 0;
  if (n_kt > t0) issue_kv(t0, 0);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();

  const int arow = tile_row(c) * QS + 8 * hh;
  const int brow = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);
  for (int t = t0; t < n_kt; ++t, buf ^= 1) {
    if (t + 1 < n_kt) issue_kv(t + 1, buf ^ 1);
    const bf16* sk = (const bf16*)(smem + C::OFF_K + buf * C::TILE_BYTES);
    const bf16* sv = (const bf16*)(smem + C::OFF_V + buf * C::TILE_BYTES);
    // S^T = K Q^T ([kv 64] x [q 32] per wave), operands read PF k-steps ahead
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
      constexpr int PF = 2;
      bf16x8 ka[C::KSD][2];
      auto ld = [&](int ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) ka[ks][mt] = *(const bf16x8*)(sk + arow + 32 * mt * QS + 16 * ks);
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) ld(ks);
#pragma unroll
      for (int ks = 0; ks < C::KSD; ++ks) {
        if (ks + PF < C::KSD) ld(ks + PF);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) s[mt] = mfma32x32x16(ka[ks][mt], qf[ks], s[mt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // visible iff key j < Lk and (causal) j <= qi: one bound per lane on the tile-local key
    const int lim = CAUSAL ? imin(Lk - 1, qi) - t * BK : Lk - 1 - t * BK;
    const int lo = qi - a.window + 1 - t * BK;  // window: first visible tile-local key
    float x[2][16];
    float tmax = -__builtin_inff();
    auto scale_mask = [&](auto masked) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          x[mt][j] = s[mt][j] * a.scale_log2;
          if constexpr (decltype(masked)::value) {
            const int kr = 32 * mt + tile_row(8 * (j >> 2) + 4 * hh + (j & 3));
            x[mt][j] = (kr <= lim && (!WINDOW || kr >= lo)) ? x[mt][j] : -__builtin_inff();
          }
          tmax = fmaxf(tmax, x[mt][j]);
        }
      }
    };
    // every key of the tile visible from every row of this wave: no element mask (wave-uniform)
    const int qmin = i0 + 32 * w, kmax = t * BK + BK - 1;
    const bool full = kmax <= Lk - 1 && (!CAUSAL || kmax <= qmin) && (!WINDOW || qmin + 31 - a.window < t * BK);
    if (full)
      scale_mask(std::false_type{});
    else
      scale_mask(std::true_type{});
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrun, tmax);
    // no visible key yet: keep everything at zero (mnew = -inf would make exp2 produce NaN)
    const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = fast_exp2(mrun - mref);  // 0 while mrun = -inf
    mrun = mnew;
    bf16x8 pk[2][2];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(x[mt][j] - mref);
        psum += p;
        pk[mt][j >> 3][j & 7] = to_bf16(p);
      }
    }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) acc[nt] *= alpha;
    // O^T += V^T P^T: k-step ksi = 2 mt + s2, k-index e is key MFMA row 16 s2 + 4 hh + e (e < 4) or
    // 16 s2 + 8 + 4 hh + e - 4 of M-tile mt; the transpose reads fetch those V rows
    {
      constexpr int NB = 4 * C::NTD, PF = 3;
      bf16x8 vt[NB];
      auto vt_load = [&](int i) {
        const int ksi = i / C::NTD, nt = i % C::NTD;
        const int o = brow + 16 * ksi * QS + 32 * nt;
        return concat(lds_read_tr4(sv + o), lds_read_tr4(sv + o + 2 * QS));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) vt[i] = vt_load(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i + PF < NB) vt[i + PF] = vt_load(i + PF);
        const int ksi = i / C::NTD, nt = i % C::NTD;
        acc[nt] = mfma32x32x16(vt[i], pk[ksi >> 1][ksi & 1], acc[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the next K/V tiles have landed
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  const float lsum = lrun + __shfl_xor(lrun, 32);
  if (qi < Lq) {
    const bool any = mrun != -__builtin_inff();  // a valid row without keys: O = 0, m = 0, l = 1
    const float inv = any ? 1.f / lsum : 0.f;
    bf16* dst = a.o + (q_start + qi) * rs + (int64_t)h * D + 4 * hh;
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const bf16x4 v4 = {to_bf16(acc[nt][4 * a4] * inv), to_bf16(acc[nt][4 * a4 + 1] * inv),
                           to_bf16(acc[nt][4 * a4 + 2] * inv), to_bf16(acc[nt][4 * a4 + 3] * inv)};
        *(bf16x4*)(dst + 32 * nt + 8 * a4) = v4;
      }
    }
    if (hh == 0) {
      const int64_t idx = (q_start + qi) * a.H + h;
      a.m[idx] = any ? mrun * (1.f / kLog2e) : 0.f;
      a.l[idx] = any ? lsum : 1.f;
    }
  }
#endif
}

// ------------------------------------------------------------------ stage 3: single-pass dQ cast

template <int D>
__global__ __launch_bounds__(256) void fa_bwd_dq_cast(const float* dq_acc, bf16* dq, int64_t total_q, int H,
                                                      float scale) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int sub = threadIdx.x % TPR;
  const int64_t pair = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;  // = t * H + h
  const int64_t t = pair / H;
  if (t >= total_q) return;
  const int h = (int)(pair - t * H);
  const float* src = dq_acc + ((int64_t)h * total_q + t) * D + sub * 8;
  const f32x4 x0 = *(const f32x4*)src;
  const f32x4 x1 = *(const f32x4*)(src + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = to_bf16(x0[e] * scale);
    r[e + 4] = to_bf16(x1[e] * scale);
  }
  *(bf16x8*)(dq + pair * D + sub * 8) = r;
}

}  // namespace fa
