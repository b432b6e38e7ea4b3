// fa_bwd_kernels.hpp -- the three device stages of the single-pass attention
// backward on gfx950:
//   fa_bwd_pre     per (token, head) row: D = rowsum(O*dO) (step 4 of the
//                  PyPTO-Gym SK-16 article's per-tile math, section 3.1),
//                  the base-2 log-sum-exp of the forward's (m, l), a zeroed
//                  fp32 dQ accumulator row, and zeroed dK/dV rows outside
//                  every sequence. HBM bound.
//   fa_bwd_main    one workgroup per (kv tile, head, sequence): keeps the
//                  tile's K, V and its fp32 dK, dV accumulators in registers,
//                  streams the q tiles through LDS and runs the five GEMMs of
//                  steps 1, 3, 6, 7, 8 on bf16 MFMA with the softmax
//                  recompute and dS (steps 2, 5) on the VALU; dQ partial sums
//                  go to the fp32 accumulator with global atomics. MFMA bound.
//   fa_bwd_dq_cast dQ = bf16(scale * accumulator). HBM bound.
#pragma once
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

// ------------------------------------------------------------------ stage 1

struct PreArgs {
  const bf16* o;
  const bf16* dout;
  const float* m;
  const float* l;
  const int* cu_q;
  const int* cu_kv;
  float* lse2;    // [H][total_q]: m*log2(e) + log2(l)
  float* dvec;    // [H][total_q]: rowsum(O*dO)
  float* dq_acc;  // [H][total_q][D]
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, batch, max_seqlen_kv, padded;
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
    float* accrow = a.dq_acc + ((int64_t)h * a.total_q + t) * D + sub * 8;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)accrow = z;
    *(f32x4*)(accrow + 4) = z;
    if (sub == 0) {
      const int64_t sidx = (int64_t)h * a.total_q + t;
      a.dvec[sidx] = acc;
      a.lse2[sidx] = a.m[pair] * kLog2e + __log2f(a.l[pair]);
    }
  }
  if (t < a.total_kv && !row_in_sequence(t, a.cu_kv, a.batch, a.padded, a.max_seqlen_kv)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *(u32x4*)(a.dk + off) = z;
    *(u32x4*)(a.dv + off) = z;
  }
}

// ------------------------------------------------------------------ stage 2

struct MainArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse2;
  const float* dvec;
  const int* cu_q;
  const int* cu_kv;
  float* dq_acc;
  bf16* dk;
  bf16* dv;
  int64_t total_q, total_kv;
  int H, batch, max_seqlen_q, max_seqlen_kv, padded, causal;
  float scale_log2;  // scale * log2(e)
  float scale;
};

template <int D>
struct MainCfg {
  static constexpr int BN = 128;       // kv rows per workgroup (32 per wave)
  static constexpr int BM = 64;        // q rows per step
  static constexpr int NW = 4;         // waves
  static constexpr int KSD = D / 16;   // MFMA k-steps over the head dim
  static constexpr int NTD = D / 32;   // 32-wide output tiles over the head dim
  static constexpr int QS = D + 8;     // LDS row stride (elements) of Q/dO tiles and of the K tile
  static constexpr int SS = BM + 8;    // LDS row stride of dS^T
  static constexpr int TPW = D / 64;   // dQ output tiles per wave
  static constexpr int NCH = BM * D / 8 / 256;  // 16-byte chunks per thread per q tile
  static constexpr int TILE = BM * QS;          // elements of one Q or dO buffer
  static constexpr int LDS_BYTES = 4 * TILE * 2 + BN * SS * 2 + 4 * BM * 4;
  static_assert(BN * QS <= 2 * TILE, "K tile must fit in the two Q buffers");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fa_bwd_main(MainArgs a) {
  using C = MainCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, QS = C::QS, SS = C::SS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  bf16* s_q = (bf16*)smem;                    // [2][BM][QS]
  bf16* s_do = s_q + 2 * C::TILE;             // [2][BM][QS]
  bf16* s_dst = s_do + 2 * C::TILE;           // [BN][SS]: dS transposed (kv-major)
  float* s_lse = (float*)(s_dst + BN * SS);   // [2][BM]
  float* s_dd = s_lse + 2 * BM;               // [2][BM]
  bf16* s_k = s_q;                            // setup only: K tile [BN][QS]

  const int HB = a.H * a.batch;
  const int tile = blockIdx.x / HB;  // heavy (low) kv tiles of every head dispatch first
  const int hb = blockIdx.x - tile * HB;
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  const int kv0 = tile * BN;
  if (kv0 >= Lk) return;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int64_t rs = (int64_t)a.H * D;  // elements between consecutive tokens
  const bf16* kb = a.k + (int64_t)h * D;
  const bf16* vb = a.v + (int64_t)h * D;
  const bf16* qb = a.q + (int64_t)h * D;
  const bf16* db = a.dout + (int64_t)h * D;

  // ---- K, V as B operands of S = Q K^T and dP = dO V^T: row kv0+32w+c, features 16ks+8hh..+7
  bf16x8 kf[C::KSD], vf[C::KSD];
  {
    const int r = kv0 + 32 * w + c;
    const int64_t gr = kv_start + r;
    const bool ok = r < Lk && gr >= 0 && gr < a.total_kv;
    const bf16x8 z = {};
#pragma unroll
    for (int ks = 0; ks < C::KSD; ++ks) {
      kf[ks] = ok ? *(const bf16x8*)(kb + gr * rs + 16 * ks + 8 * hh) : z;
      vf[ks] = ok ? *(const bf16x8*)(vb + gr * rs + 16 * ks + 8 * hh) : z;
    }
  }
  // ---- K tile through LDS, then K^T fragments (B operand of dQ = dS K) for this wave's feature slice
  for (int ch = tid; ch < BN * D / 8; ch += 256) {
    const int r = ch / (D / 8), col = (ch % (D / 8)) * 8;
    const int64_t gr = kv_start + kv0 + r;
    const bool ok = kv0 + r < Lk && gr >= 0 && gr < a.total_kv;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *(u32x4*)(s_k + r * QS + col) = ok ? *(const u32x4*)(kb + gr * rs + col) : z;
  }
  __syncthreads();
  const int ntq = (w * C::TPW) >> 1;  // this wave's 32-wide feature slice of dQ
  bf16x8 ktf[BN / 16];
  {
    const int col = 32 * ntq + 16 * (g & 1) + 4 * (gi & 3);
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const int r0 = 16 * ks + 8 * hh + (gi >> 2);
      ktf[ks] = concat(lds_read_tr4(s_k + r0 * QS + col), lds_read_tr4(s_k + (r0 + 4) * QS + col));
    }
  }
  __syncthreads();

  f32x16 accK[C::NTD], accV[C::NTD];
#pragma unroll
  for (int nt = 0; nt < C::NTD; ++nt) {
    accK[nt] = f32x16{};
    accV[nt] = f32x16{};
  }

  const int n_qt = (Lq + BM - 1) / BM;
  int qt = a.causal ? kv0 / BM : 0;

  // global -> registers for q tile `t`
  u32x4 pq[C::NCH], pd[C::NCH];
  float pst = 0.f;
  auto fetch = [&](int t) {
    const int i0 = t * BM;
#pragma unroll
    for (int u = 0; u < C::NCH; ++u) {
      const int ch = tid + 256 * u;
      const int r = ch / (D / 8), col = (ch % (D / 8)) * 8;
      const int64_t gr = q_start + i0 + r;
      const bool ok = i0 + r < Lq && gr >= 0 && gr < a.total_q;
      const u32x4 z = {0u, 0u, 0u, 0u};
      pq[u] = ok ? *(const u32x4*)(qb + gr * rs + col) : z;
      pd[u] = ok ? *(const u32x4*)(db + gr * rs + col) : z;
    }
    if (tid < 2 * BM) {
      const int r = tid & (BM - 1);
      const int64_t gr = q_start + i0 + r;
      const bool ok = i0 + r < Lq && gr >= 0 && gr < a.total_q;
      const float* src = tid < BM ? a.lse2 : a.dvec;
      pst = ok ? src[(int64_t)h * a.total_q + gr] : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < C::NCH; ++u) {
      const int ch = tid + 256 * u;
      const int r = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *(u32x4*)(s_q + buf * C::TILE + r * QS + col) = pq[u];
      *(u32x4*)(s_do + buf * C::TILE + r * QS + col) = pd[u];
    }
    if (tid < 2 * BM) (tid < BM ? s_lse : s_dd)[buf * BM + (tid & (BM - 1))] = pst;
  };

  int buf = 0;
  if (qt < n_qt) {
    fetch(qt);
    stash(0);
  }
  __syncthreads();

  const int jcol = kv0 + 32 * w + c;  // this lane's key row (sequence-local) in S and dP
  for (; qt < n_qt; ++qt, buf ^= 1) {
    const bool has_next = qt + 1 < n_qt;
    if (has_next) fetch(qt + 1);
    const int i0 = qt * BM;
    const bf16* sq = s_q + buf * C::TILE;
    const bf16* sd = s_do + buf * C::TILE;

    // steps 1 and 3: S = Q K^T, dP = dO V^T  ([q 64] x [kv 32] per wave)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      dp[mt] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < C::KSD; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 qa = *(const bf16x8*)(sq + (32 * mt + c) * QS + 16 * ks + 8 * hh);
        const bf16x8 da = *(const bf16x8*)(sd + (32 * mt + c) * QS + 16 * ks + 8 * hh);
        s[mt] = mfma32x32x16(qa, kf[ks], s[mt]);
        dp[mt] = mfma32x32x16(da, vf[ks], dp[mt]);
      }
    }

    // steps 2 and 5: P = exp2(S*scale*log2e - lse2), masked; dS = P (dP - D); both to bf16
    const bool edge = (i0 + BM > Lq) || (kv0 + BN > Lk) || (a.causal && i0 < kv0 + BN - 1);
    bf16x8 pk[2][2], dsk[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int rloc = 32 * mt + 8 * a4 + 4 * hh;
        const f32x4 lse = *(const f32x4*)(s_lse + buf * BM + rloc);
        const f32x4 dd = *(const f32x4*)(s_dd + buf * BM + rloc);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int j = 4 * a4 + bb;
          float p = fast_exp2(s[mt][j] * a.scale_log2 - lse[bb]);
          if (edge) {
            const int i = i0 + rloc + bb;
            const bool vis = i < Lq && jcol < Lk && (!a.causal || jcol <= i);
            p = vis ? p : 0.f;
          }
          const float ds = p * (dp[mt][j] - dd[bb]);
          pk[mt][j >> 3][j & 7] = to_bf16(p);
          dsk[mt][j >> 3][j & 7] = to_bf16(ds);
        }
      }
    }
    // dS^T to LDS: row = this lane's key, 4 consecutive queries per store
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const bf16x8 src = dsk[mt][a4 >> 1];
        const int o4 = 4 * (a4 & 1);
        const bf16x4 v4 = {src[o4], src[o4 + 1], src[o4 + 2], src[o4 + 3]};
        *(bf16x4*)(s_dst + (32 * w + c) * SS + 32 * mt + 8 * a4 + 4 * hh) = v4;
      }
    }

    // steps 7 and 6: dV += P^T dO, dK += dS^T Q  (scale applied at write-back)
#pragma unroll
    for (int nt = 0; nt < C::NTD; ++nt) {
      const int col = 32 * nt + 16 * (g & 1) + 4 * (gi & 3);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r0 = 32 * mt + 16 * s2 + 4 * hh + (gi >> 2);
          const bf16x8 bdo = concat(lds_read_tr4(sd + r0 * QS + col), lds_read_tr4(sd + (r0 + 8) * QS + col));
          const bf16x8 bq = concat(lds_read_tr4(sq + r0 * QS + col), lds_read_tr4(sq + (r0 + 8) * QS + col));
          accV[nt] = mfma32x32x16(pk[mt][s2], bdo, accV[nt]);
          accK[nt] = mfma32x32x16(dsk[mt][s2], bq, accK[nt]);
        }
      }
    }
    __syncthreads();  // dS^T complete

    // step 8: dQ partial = dS K over this tile's 128 keys, added to the fp32 accumulator
#pragma unroll
    for (int tt = 0; tt < C::TPW; ++tt) {
      const int mtq = (w * C::TPW + tt) & 1;
      const int col = 32 * mtq + 16 * (g & 1) + 4 * (gi & 3);
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const int r0 = 16 * ks + 8 * hh + (gi >> 2);
        const bf16x8 af = concat(lds_read_tr4(s_dst + r0 * SS + col), lds_read_tr4(s_dst + (r0 + 4) * SS + col));
        acc = mfma32x32x16(af, ktf[ks], acc);
      }
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int i = i0 + 32 * mtq + 8 * a4 + 4 * hh + bb;
          const int64_t gr = q_start + i;
          if (i < Lq && gr >= 0 && gr < a.total_q)
            unsafeAtomicAdd(a.dq_acc + ((int64_t)h * a.total_q + gr) * D + 32 * ntq + c, acc[4 * a4 + bb]);
        }
      }
    }
    if (has_next) stash(buf ^ 1);
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
        const int64_t gr = kv_start + r;
        if (r < Lk && gr >= 0 && gr < a.total_kv) {
          const int64_t o = gr * rs + (int64_t)h * D + 32 * nt + c;
          a.dk[o] = to_bf16(accK[nt][4 * a4 + bb] * a.scale);
          a.dv[o] = to_bf16(accV[nt][4 * a4 + bb]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ stage 3

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
