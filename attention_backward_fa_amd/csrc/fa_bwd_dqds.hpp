// fa_bwd_dqds.hpp -- dQ of the stored-dS form: dQ = scale * dS K (step 8 of the per-tile math of the
// PyPTO-Gym SK-16 article, section 3.1) from the dS the dK/dV kernel wrote, so that S and dP are not
// formed a second time: the 64-key kernel's blocks (head dims of 128) or the wide-head kernel's pieces
// (PIECES, a head dim above 128).
//
// A dS block holds one 32-row q step against one 256-key kv tile (16 KB of bf16) in the order the dK/dV
// kernel's lanes hold the values: piece ((w * 2 + n) * 2 + s2) of 1 KB holds, at lane l = c + 32 hh,
// the 16 bytes of key 64 w + 32 n + c at positions 16 hh + 8 s2 ..+7, and position p stands for query
// row 32 t + tile_row(8 ((p & 15) >> 2) + 4 (p >> 4) + (p & 3)) of step t. Every store of the writer
// and every load of the reader then covers whole 1 KB runs. Block (t, j) of (sequence b, query head h)
// sits at ds + (((b H + h) nkt + j) nqs + t) * 8192 elements (a writer workgroup, one kv tile, writes
// its steps' blocks one after another), for the nqs steps and nkt tiles of the longest sequences;
// steps and tiles outside those are neither written nor read. A dS piece (ds_piece) holds a 32-row q step
// against a 32-key tile, 2 KB in the order of the wide-head kernel's lanes: half s2 (1 KB) holds, at lane
// c + 32 hh, the 16 bytes of key c at positions 16 hh + 8 s2 ..+7, the positions standing for query rows
// as in a block; piece (t, kt) of (sequence b, query head h) starts at element ds_piece(b * H + h, kt, t).
//
// One workgroup of four waves per (128-row q tile, head, sequence), two per CU; wave w takes q step
// 4 * tile + w. Per 64-key step a wave loads its 64 x 32 dS values straight into registers (16 bytes
// per lane per 32 x 16 piece, in the A-operand layout of an MFMA whose rows are keys), two steps ahead,
// transposes them with two MFMAs against identity B operands per 32-key tile (exact: one product per
// output, by 1), and accumulates dQ^T += K^T dS^T with K from an LDS tile, as the recompute form's dQ
// kernel does. Under a causal mask, a wave reading pieces stops at its own diagonal (key tiles kt <= t):
// the wide-head kernel's steps start at the q step of its 64-key tile's first key, so a piece past a
// wave's diagonal may not have been written (it holds no visible pair); a block is written whole for
// every step a kv tile's workgroup runs.
#pragma once
#include "fa_bwd_kernels.hpp"

namespace fa {

// NW_ waves, one 32-row q step each: four (two workgroups per CU), or eight (one per CU; each K tile
// brought to LDS serves twice the rows, half the transfers from L2)
template <int DQ, int NW_ = 4>
struct DqDsCfg {
  static constexpr int D = DQ;               // the Q/K head dim, padded to a multiple of 32
  static constexpr int NW = NW_, NT = 64 * NW;
  static constexpr int BQ = 32 * NW;         // q rows per workgroup
  static constexpr int BK = 64;              // keys per step
  static constexpr int QS = D + 8;           // padded row stride of the K tile
  static constexpr int CPR = QS / 8;
  static constexpr int TK_BYTES = BK * QS * 2;
  static constexpr int NDMA_K = TK_BYTES / 1024;
  static constexpr int NTQ = D / 32;         // 32-wide feature tiles of dQ^T
  static constexpr int BLOCK = 256 * 32;     // elements of one dS block
  static constexpr int LDS_BYTES = 2 * TK_BYTES;
  static_assert(DQ % 32 == 0 && DQ <= 256, "padded head dims");
  static_assert(TK_BYTES % 1024 == 0, "whole 1 KB transfers");
};

// EXACT: the Q/K head dim equals DQ (else a.d_qk, padded to DQ); PIECES: the wide-head kernel's pieces
// (no window), else the 64-key kernel's blocks
template <int DQ, bool EXACT, bool PIECES, bool CAUSAL, bool WINDOW, int NW = 4>
__global__ __attribute__((amdgpu_flat_work_group_size(DqDsCfg<DQ, NW>::NT, DqDsCfg<DQ, NW>::NT),
                          amdgpu_waves_per_eu(2, 2)))
void fa_bwd_dq_ds(MainArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = DqDsCfg<DQ, NW>;
  constexpr int BQ = C::BQ, BK = C::BK, QS = C::QS, D = C::D, NTQ = C::NTQ;
  static_assert(CAUSAL || !WINDOW, "a window implies the causal bound");
  static_assert(!PIECES || !WINDOW, "pieces are stored without a window");
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
  const int dqk = EXACT ? D : a.d_qk;
  const int64_t rsq = (int64_t)a.H * dqk, rskq = (int64_t)a.Hk * dqk;  // row strides of dQ and of K
  const int rskqb = (int)(rskq * 2);
  const int hk = h / (a.H / a.Hk);
  const bf16* kb = a.k + kv_start * rskq + (int64_t)hk * dqk;
  const int t = qtile * NW + w;  // this wave's 32-row q step
  // the wave's dS blocks (one per 256-key kv tile) or pieces (one per 32-key tile). A step whose rows
  // all lie past the sequence has none (past the longest sequence, none inside the workspace): its loads
  // read an empty range.
  const bool t_rows = 32 * t < Lq && t < a.ds_nqs;
  const bf16* dsb = a.ds + (PIECES ? ds_piece(a, hb, 0, t_rows ? t : 0)
                                   : ((int64_t)hb * a.ds_nkt * a.ds_nqs + (t_rows ? t : 0)) * C::BLOCK);
  // from a kv tile's block (a key tile's piece) to the next's
  const int64_t tile_stride = (int64_t)a.ds_nqs * (PIECES ? kDsPiece : C::BLOCK);

  // 64-key steps: under a causal mask up to the last row's diagonal (the blocks of those keys were
  // written whole, with zeros where a row does not see a key)
  int n_kt = (Lk + BK - 1) / BK;
  if (CAUSAL) n_kt = imin(n_kt, (i0 + BQ - 1) / BK + 1);
  // window: from the first key the tile's first row sees. The dK/dV kernel's workgroup of kv tile j
  // wrote the blocks of q steps up to the last row that sees one of its keys, (256 j + 254 + window) / 32
  // (all others of this wave's blocks would hold zeros only): past it this wave reads an empty range.
  const int t0 = WINDOW ? imax(0, i0 - a.window + 1) / BK : 0;

  {  // zero the K buffers once (rows past the sequence must be finite)
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
  // dS of step s: for key tile m (32 keys) and k-step e (16 positions), this lane's 16 bytes: key
  // 64 s + 32 m + tile_row(c), positions 16 e + 8 hh ..+7, i.e. lane tile_row(c) + 32 e of piece
  // ((s % 4) * 2 + m) * 2 + hh of block s / 4, or of half hh of piece (t, 2 s + m). Keys past the
  // sequence, steps past the last and (pieces) key tiles past the wave's diagonal read as zeros.
  auto load_ds = [&](int s, bf16x8 (&x)[2][2]) {
    if constexpr (PIECES) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int kt = 2 * s + m;
        const bool live = t_rows && s < n_kt && kt < a.ds_nkt && (!CAUSAL || kt <= t);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(dsb + kt * tile_stride, live ? kDsPiece * 2 : 0);
        const bool key_in = 32 * kt + tile_row(c) < Lk;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int off = (hh * 512 + (tile_row(c) + 32 * e) * 8) * 2;
          x[m][e] = __builtin_bit_cast(bf16x8, buf_load16(rs, key_in ? off : kOutOfRange));
        }
      }
    } else {
      const int j = s >> 2, wp = s & 3;
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(dsb + j * tile_stride, t_rows && s < n_kt && j < a.ds_nkt &&
                                               (!WINDOW || 32 * t <= 256 * j + 254 + a.window) ? C::BLOCK * 2 : 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bool key_in = 256 * j + 64 * wp + 32 * m + tile_row(c) < Lk;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int off = ((((wp * 2 + m) * 2 + hh) * 512) + (tile_row(c) + 32 * e) * 8) * 2;
          x[m][e] = __builtin_bit_cast(bf16x8, buf_load16(rs, key_in ? off : kOutOfRange));
        }
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
  issue_k(t0, t0 & 1);
  load_ds(t0, ds0);
  load_ds(t0 + 1, ds1);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // three register sets for the dS of steps s, s + 1, s + 2 (each step prefetches into the one the
  // step before it has used)
  for (int s = t0; s < n_kt; s += 3) {
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
