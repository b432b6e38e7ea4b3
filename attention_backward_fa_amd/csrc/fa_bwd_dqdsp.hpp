// fa_bwd_dqdsp.hpp -- dQ of the stored-dS form for the wide-head kernels: dQ = scale * dS K (step 8 of
// the per-tile math of the PyPTO-Gym SK-16 article, section 3.1) from the dS pieces the wide-head dK/dV
// kernel wrote, so that S and dP (at head dims above 128) are not formed a second time.
//
// A dS piece holds a 32-row q step against a 32-key tile, 2 KB of bf16 in the order the dK/dV kernel's
// lanes hold the values after its softmax: half s2 (1 KB) holds, at lane l = c + 32 hh, the 16 bytes of
// key c at positions 16 hh + 8 s2 ..+7, and position p stands for query row
// tile_row(8 ((p & 15) >> 2) + 4 (p >> 4) + (p & 3)) of the step. Piece (t, kt) of (sequence b, query
// head h) starts at element ds_piece(b * H + h, kt, t): a dK/dV wave writes the pieces of its key tile
// one step after another. Pieces of steps and key tiles past the longest sequences are neither written
// nor read.
//
// One workgroup of four waves per (128-row q tile, head, sequence), two per CU; wave w takes q step
// 4 * tile + w. Per 64-key step a wave loads its two pieces straight into registers (16 bytes per lane
// per 32 x 16 half: the A-operand layout of an MFMA whose rows are keys), two steps ahead, transposes
// each with two MFMAs against identity B operands (exact: one product per output, by 1), and
// accumulates dQ^T += K^T dS^T with K from an LDS tile, as the recompute form's dQ kernel does. Under a
// causal mask a wave reads the key tiles up to its own diagonal (kt <= t): the dK/dV kernel writes every
// piece of a step it runs, masked pairs as zeros, and its steps start at the q step of its tile's first
// key, so every piece at or below a wave's diagonal was written (those above hold no visible pair).
#pragma once
#include "fa_bwd_kernels.hpp"

namespace fa {

template <int DQ>
struct DqDspCfg {
  static constexpr int NW = 4, NT = 64 * NW;
  static constexpr int BQ = 32 * NW;          // q rows per workgroup
  static constexpr int BK = 64;               // keys per step
  static constexpr int QS = DQ + 8;           // padded row stride of the K tile
  static constexpr int CPR = QS / 8;
  static constexpr int TK_BYTES = BK * QS * 2;
  static constexpr int NDMA_K = TK_BYTES / 1024;
  static constexpr int NTQ = DQ / 32;         // 32-wide feature tiles of dQ^T
  static constexpr int LDS_BYTES = 2 * TK_BYTES;
  static_assert(DQ % 32 == 0 && DQ <= 256, "padded head dims");
  static_assert(TK_BYTES % 1024 == 0, "whole 1 KB transfers");
};

// EXACT: the head dim of Q and K equals DQ (else a.d_qk, padded to DQ)
template <int DQ, bool EXACT, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(DqDspCfg<DQ>::NT, DqDspCfg<DQ>::NT), amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_dsp(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqDspCfg<DQ>;
  constexpr int BQ = C::BQ, BK = C::BK, QS = C::QS, NTQ = C::NTQ;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  // work item: as the recompute form's dQ kernel (host schedule, head-major per XCD, or tile-major with
  // the q tiles that see the most keys first)
  const int HB = a.H * a.batch;
  const int n_qt_max = (a.max_seqlen_q + BQ - 1) / BQ;
  int tr, hb;
  if (a.sched) {
    tr = 0;
    hb = a.sched[2 * blockIdx.x + 1];
  } else if (a.head_major) {
    const int x = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int k = slot / n_qt_max;
    tr = slot - k * n_qt_max;
    hb = x + 8 * k;
  } else {
    tr = blockIdx.x / HB;
    hb = blockIdx.x - tr * HB;
  }
  const int b = hb / a.H, h = hb - (hb / a.H) * a.H;
  int64_t q_start, kv_start;
  int Lq, Lk;
  seq_of(a.cu_q, b, a.padded, a.max_seqlen_q, q_start, Lq);
  seq_of(a.cu_kv, b, a.padded, a.max_seqlen_kv, kv_start, Lk);
  Lq = clamp_len(q_start, Lq, a.total_q);
  Lk = clamp_len(kv_start, Lk, a.total_kv);
  const int qtile = a.sched ? a.sched[2 * blockIdx.x] : CAUSAL ? n_qt_max - 1 - tr : tr;
  const int i0 = qtile * BQ;
  if (i0 >= Lq) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, c = lane & 31, g = lane >> 4, gi = lane & 15;
  const int dqk = EXACT ? DQ : a.d_qk;
  const int64_t rsq = (int64_t)a.H * dqk, rskq = (int64_t)a.Hk * dqk;  // row strides of dQ and of K
  const int rskqb = (int)(rskq * 2);
  const int hk = h / (a.H / a.Hk);
  const bf16* kb = a.k + kv_start * rskq + (int64_t)hk * dqk;
  const int t = qtile * 4 + w;  // this wave's 32-row q step
  // the wave's dS pieces (one per 32-key tile). A step whose rows all lie past the sequence has no
  // pieces (past the longest sequence, none inside the workspace): its loads read an empty range.
  const bool t_rows = 32 * t < Lq && t < a.ds_nqs;
  const bf16* dsb = a.ds + ds_piece(a, hb, 0, t_rows ? t : 0);
  const int64_t kt_stride = (int64_t)a.ds_nqs * kDsPiece;  // from a key tile's piece to the next's

  // 64-key steps: under a causal mask up to the last row's diagonal
  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);

  {  // zero the K buffers once (rows past the sequence and features past the head dim must be zeros)
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int o = tid * 16; o < C::LDS_BYTES; o += C::NT * 16) *(u32x4*)(smem + o) = z;
  }
  __syncthreads();

  // K tile of step s into buffer bi: transfers w, w + 4, ... of 1 KB, untracked (the step's LDS reads
  // of the other buffer must not wait for them; the end-of-step wait and barrier order them)
  constexpr int NJ = (C::NDMA_K + C::NW - 1) / C::NW;
  int offk[NJ];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) offk[jj] = tile_dma_off(w + C::NW * jj, lane, C::CPR, rskqb, dqk);
  auto issue_k = [&](int s, int bi) {
    const int j0 = s * BK, rows = s < n_kt ? imin(Lk - j0, BK) : 0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (int64_t)j0 * rskq, (int64_t)rows * rskqb);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = w + C::NW * jj;
      if (j < C::NDMA_K)
        dma16_untracked(rk, offk[jj], (__attribute__((address_space(3))) void*)(smem + bi * C::TK_BYTES + 1024 * j));
    }
  };
  // dS of step s: for key tile kt = 2 s + m (32 keys) and k-step e (16 positions), this lane's 16
  // bytes: key 32 kt + tile_row(c), positions 16 e + 8 hh ..+7, i.e. lane tile_row(c) + 32 e of half hh
  // of piece (t, kt). Keys past the sequence, key tiles past the wave's diagonal and steps past the last
  // read as zeros.
  auto load_ds = [&](int s, bf16x8 (&x)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int kt = 2 * s + m;
      const bool live = t_rows && s < n_kt && kt < a.ds_nkt && (!CAUSAL || kt <= t);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(dsb + kt * kt_stride, live ? kDsPiece * 2 : 0);
      const bool key_in = 32 * kt + tile_row(c) < Lk;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int off = (hh * 512 + (tile_row(c) + 32 * e) * 8) * 2;
        x[m][e] = __builtin_bit_cast(bf16x8, buf_load16(rs, key_in ? off : kOutOfRange));
      }
    }
  };
  // identity B operands: element jj of this lane is 1 where position c = 16 e + 8 hh + jj
  bf16x8 eye[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) eye[e][jj] = to_bf16(c == 16 * e + 8 * hh + jj ? 1.f : 0.f);

  f32x16 acc[NTQ];
#pragma unroll
  for (int nt = 0; nt < NTQ; ++nt) acc[nt] = f32x16{};

  const int browk = (hh + 4 * (gi >> 2)) * QS + 16 * (g & 1) + 4 * (gi & 3);
  // step s: dS^T of the step's two key tiles is formed in the layout of an MFMA result (rows: keys
  // tile_row(r), column: position c) and used as the bf16 B operand of dQ^T += K^T dS^T; then the K tile
  // of s + 1 and the dS of s + 2 load. The loads issue on every step, with empty ranges past the last
  // (no memory is read), so that the same loads precede every use of a register set and the waits for
  // them count exactly; steps past the last skip their arithmetic.
  auto step = [&](int s, const bf16x8 (&dc)[2][2], bf16x8 (&dpf)[2][2]) {
    const bool live = s < n_kt;
    const bf16* sk = (const bf16*)(smem + (s & 1) * C::TK_BYTES);
    bf16x8 dsk[2][2];
    if (live) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x16 tt = f32x16{};
        tt = mfma32x32x16(dc[m][0], eye[0], tt);
        tt = mfma32x32x16(dc[m][1], eye[1], tt);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) dsk[m][jj >> 3][jj & 7] = to_bf16(tt[jj]);
      }
    }
    // after the transposes have read this step's dS registers: a load issued earlier would make the
    // wait for them wait for it too
    __builtin_amdgcn_sched_barrier(0);
    issue_k(s + 1, (s + 1) & 1);
    load_ds(s + 2, dpf);
    __builtin_amdgcn_sched_barrier(0);
    if (live) {
      constexpr int NB = 4 * NTQ, PF = 3;
      bf16x8 kt[NB];
      auto kt_load = [&](int i) {
        const int ksi = i / NTQ, nt = i % NTQ;
        const int o = browk + 16 * ksi * QS + 32 * nt;
        return concat(lds_read_tr4(sk + o), lds_read_tr4(sk + o + 2 * QS));
      };
#pragma unroll
      for (int i = 0; i < PF; ++i) kt[i] = kt_load(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (i + PF < NB) kt[i + PF] = kt_load(i + PF);
        const int ksi = i / NTQ, nt = i % NTQ;
        acc[nt] = mfma32x32x16(kt[i], dsk[ksi >> 1][ksi & 1], acc[nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the K tile of s + 1 has landed: loads complete in order, and only the four dS loads issued after
    // it may still be in flight
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  bf16x8 ds0[2][2], ds1[2][2], ds2[2][2];
  issue_k(0, 0);
  load_ds(0, ds0);
  load_ds(1, ds1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // three register sets for the dS of steps s, s + 1, s + 2 (each step prefetches into the one the
  // step before it has used)
  for (int s = 0; s < n_kt; s += 3) {
    step(s, ds0, ds2);
    step(s + 1, ds1, ds0);
    step(s + 2, ds2, ds1);
  }

  // dQ = scale * (dQ^T)^T in bf16: this lane holds features 32 nt + 8 a4 + 4 hh + bb of position c
  const int p = c;
  const int qi = 32 * t + tile_row(8 * ((p & 15) >> 2) + 4 * (p >> 4) + (p & 3));
  if (qi < Lq) {
    bf16* dst = a.dq + (q_start + qi) * rsq + (int64_t)h * dqk + 4 * hh;
#pragma unroll
    for (int nt = 0; nt < NTQ; ++nt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        if (32 * nt + 8 * a4 + 4 * hh >= dqk) continue;  // head dims are multiples of 8
        const bf16x4 v4 = {to_bf16(acc[nt][4 * a4] * a.scale), to_bf16(acc[nt][4 * a4 + 1] * a.scale),
                           to_bf16(acc[nt][4 * a4 + 2] * a.scale), to_bf16(acc[nt][4 * a4 + 3] * a.scale)};
        *(bf16x4*)(dst + 32 * nt + 8 * a4) = v4;
      }
    }
  }
#endif
}

}  // namespace fa
