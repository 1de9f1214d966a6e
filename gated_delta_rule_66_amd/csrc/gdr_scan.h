// gdr_scan.h -- the sequential inter-chunk state recurrence (forward
// direction) and its intra-GPU context-parallel (CP) split.
//
// One workgroup = 4 waves = one (sequence, value head, T-segment, column
// block).  The state S (K x V fp32) is split by value columns: the columns
// of S evolve independently, so a workgroup owns CW = 64 * VB of them and
// wave w owns 16 * VB, kept as MFMA accumulators for the whole segment.
// Per chunk (gamma = g_cum, L = last valid row):
//   R     = diag(beta) V - diag(beta e^gamma) (K S)
//   Delta = A R                                         (WY form)
//   O     = scale (diag(e^gamma) (Q S) + P Delta),   P = lower_incl(Q K^T o Gamma)
//   S     = e^{gamma_L} S + K^T (diag(e^{gamma_L - gamma}) Delta)
// The next chunk's tiles are loaded into registers while the current chunk
// computes.
//
// Intra-GPU context parallelism (the pages' "intra-card CP"; the mechanism is
// ours): a chunk maps its start state affinely, S' = T_c S + B_c with
// T_c = e^{gamma_L} I - K~^T A X and B_c = K~^T A Y.  So a segment of chunks
// maps S_start to S_end = T_seg S_start + B_seg, and (T_seg | B_seg) is the
// end state of the same recurrence run on the augmented K x 2V state
// [I | 0] with values [0 | V] (MODE_AUG).  Pass 1 computes the transitions of
// every segment but the last in parallel, pass 2 (cp_combine_kernel) chains
// the segment start states, pass 3 reruns each segment from its start state
// with outputs.  The plan depends only on shapes.
#pragma once

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

// MODE_OUT: outputs; MODE_OUT_H: outputs and the chunk-start states h;
// MODE_AUG: segment transitions; MODE_STATE: chunk-start states only.
enum ScanMode { MODE_OUT = 0, MODE_AUG = 1, MODE_STATE = 2, MODE_OUT_H = 3 };

// Chunk offsets of packed sequences, computed on the device so that no
// device-to-host copy is needed: offs[0] = 0, offs[n+1] = offs[n] +
// ceil(len_n / 64); and order[k] = the sequence of rank k by chunk count,
// longest first (ties by index), each thread ranking its sequences against
// all others.
static __global__ void chunk_offsets_kernel(const int32_t* cu, int N, int32_t* offs,
                                            int32_t* order) {
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    offs[0] = 0;
    for (int n = 0; n < N; ++n) {
      acc += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
      offs[n + 1] = acc;
    }
  }
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int32_t cn = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const int32_t cm = (cu[m + 1] - cu[m] + kChunk - 1) / kChunk;
      rank += (cm > cn || (cm == cn && m < n)) ? 1 : 0;
    }
    order[rank] = n;
  }
}

struct ScanArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const float* gcum;
  const void* A;
  const float* h0;        // [N, Hv, K, V] (or [.., V, K] when svf), nullable
  void* o;                // MODE_OUT output
  void* h;                // chunk-start states (in_dtype), nullable
  float* ht;              // final state, nullable
  const float* seg_start; // [units, P, K, V] fp32 segment start states (P > 1)
  float* seg_out;         // [units, P, K, 2V] fp32 augmented end states (pass 1)
  // [units, P, K, K] fp32 segment transitions T_seg kept for the backward
  // (nullable).  Forward: pass 1 writes T_seg here instead of into seg_out
  // and pass 2 reads it back.  Backward (reverse): pass 2 applies the
  // forward's T_seg transposed, which is the state gradient's transition.
  float* trans;
  const int32_t* cu;
  const int32_t* offs;
  const int32_t* order;  // packed input: sequences by chunk count, longest first (block_pos)
  int N, T, Hq, Hv;
  int nc_dense;
  int P;    // segments per sequence
  int nvs;  // column blocks per (unit, segment)
  float scale;
  int svf;     // layout of h0 / ht / user h
  int h_svf;   // layout of h: the user's h follows svf; MODE_STATE always writes [V][K]
  int h_vm;    // h in the packed layout (packed_off) whatever svf says: the
               // states the forward keeps for the backward.  The output pass's
               // launch choice follows this, never svf, so both state layouts
               // run the same kernel.
  int reverse; // cp_combine_kernel: chain segments backwards (state gradients)
  int qk_norm; // q, k rows scaled to unit length before use
  int beta_mode; // bit 0 sigmoid of a beta logit, bit 1 twice beta
};

// Chunks [c0, c1) of segment p; the segment holding the last chunk is
// p_last (0 for an empty sequence).
struct SegRange {
  int c0, c1, p_last;
};
__device__ __forceinline__ SegRange seg_range(int nch, int P, int p) {
  SegRange r;
  const int sc = (nch + P - 1) / P;
  r.c0 = min(p * sc, nch);
  r.c1 = min(r.c0 + sc, nch);
  r.p_last = (nch == 0) ? 0 : (nch - 1) / sc;
  return r;
}

// Index of the upper-triangular tile (ib, rb), ib <= rb, of P^T in a packed
// list of ten tiles.
__host__ __device__ constexpr int tri_idx(int ib, int rb) { return rb * (rb + 1) / 2 + ib; }

// One workgroup's share of a scan pass: block b of the pass's nb (block_pos
// gives its unit).  A device function so that two independent passes can
// share one launch (the backward's state and state-gradient scans).
template <typename T, int VB, int MODE>
__device__ __forceinline__ void scan_body(const ScanArgs& a, int b, int nb) {
  typedef typename VT<T>::x8 x8;
  constexpr int CW = 64 * VB;          // columns per workgroup
  constexpr int LD = 136;              // q / k tile leading dimension
  constexpr int LDV = CW + 8;          // v tile leading dimension
  constexpr int LDA = 72;              // A tile leading dimension
  constexpr bool OUT = (MODE == MODE_OUT || MODE == MODE_OUT_H);
  constexpr bool HOUT = (MODE == MODE_STATE || MODE == MODE_OUT_H);  // writes h
  constexpr bool HST = (MODE == MODE_OUT_H);  // may stage h in LDS (key-major h)
  __shared__ __align__(16) T Ks[64 * LD];
  __shared__ __align__(16) T Qs[OUT ? 64 * LD : 8];
  __shared__ __align__(16) T Vs[64 * LDV];
  __shared__ __align__(16) T As[64 * LDA];
  __shared__ __align__(16) T Hs[HST ? 128 * (CW + 8) : 8];
  __shared__ __align__(16) float gam[64], bet[64], eg[64], bex[64], dl[64];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const BlockPos bp = block_pos(a.order, b, nb, a.P * a.nvs, a.Hv);
  const int vs = bp.sub % a.nvs;
  const int p = bp.sub / a.nvs, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const SegRange sr = seg_range(nch, a.P, p);
  const int cb0 = vs * CW;
  const bool isT = (MODE == MODE_AUG) && cb0 < kDim;  // transition columns
  if (MODE == MODE_AUG) {
    if (p >= sr.p_last) return;   // the last segment needs no transition
    if (p == 0 && isT) return;    // segment 0 starts from h0: its end state suffices
  } else {
    if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;  // empty segment
  }
  const int vcol0 = (MODE == MODE_AUG) ? (isT ? 0 : cb0 - kDim) : cb0;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const int64_t KV = (int64_t)kDim * kDim;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  const T* Ag = reinterpret_cast<const T*>(a.A);
  const T* beta = reinterpret_cast<const T*>(a.beta);
  const int cw0 = 16 * VB * w;  // this wave's first column inside the block

  // ---- initial state: h0 (segment 0) or the chained segment start; every
  // load is issued before the first is used (a null source reads zeros) ----
  f32x4 S[8][VB];
  if (MODE == MODE_AUG && isT) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S[kb][vb][e] = (16 * kb + 4 * grp + e == cb0 + cw0 + 16 * vb + col) ? 1.f : 0.f;
  } else {
    // the value columns of an inner segment's transition start from zero
    // (their end state is B_seg); its start state is not known before pass 2
    const float* src = (p == 0) ? (a.h0 ? a.h0 + unit * KV : nullptr)
                       : (MODE == MODE_AUG) ? nullptr
                                            : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == 0) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = vcol0 + cw0 + 16 * vb + col;
          S[kb][vb][e] = buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
        }
  }

  // ---- register prefetch of one chunk ----
  TileRegs<128, 256> rq, rk;
  TileRegs<CW, 256> rv;
  TileRegs<64, 256> ra;
  float r_g = 0.f, r_gl = 0.f;
  T r_b = from_f<T>(0.f);  // raw bits: converting here would wait for every prefetched load
  auto prefetch = [&](int c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    if (OUT) tile_load<T, 128, 256>(rq, q + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc);
    tile_load<T, 128, 256>(rk, k + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc);
    if (!isT) tile_load<T, CW, 256>(rv, v + (t0 * a.Hv + h) * kDim + vcol0, (int64_t)a.Hv * kDim, Cc);
    tile_load<T, 64, 256>(ra, Ag + (t0 * a.Hv + h) * kChunk, (int64_t)a.Hv * kChunk, Cc);
    if (tid < 64) {
      r_g = a.gcum[(t0 + min(tid, Cc - 1)) * a.Hv + h];
      r_gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
      r_b = (tid < Cc) ? beta[(t0 + tid) * a.Hv + h] : from_f<T>(0.f);
    }
  };

  __builtin_amdgcn_s_waitcnt(0);  // the initial state is in (see scan_out_kernel)
  if (sr.c0 < sr.c1) prefetch(sr.c0);
  for (int c = sr.c0; c < sr.c1; ++c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    if (a.qk_norm) {
      if (OUT) l2norm_rows<T, 256>(rq, nullptr);
      l2norm_rows<T, 256>(rk, nullptr);
    }
    __syncthreads();  // the previous chunk is done with LDS
    if (OUT) tile_store<T, 128, 256>(Qs, LD, rq);
    tile_store<T, 128, 256>(Ks, LD, rk);
    if (!isT) tile_store<T, CW, 256>(Vs, LDV, rv);
    tile_store<T, 64, 256>(As, LDA, ra);
    if (tid < 64) {
      const float bv = tid < Cc ? beta_used(to_f(r_b), a.beta_mode) : 0.f;
      gam[tid] = r_g;
      bet[tid] = bv;
      const float e = __expf(r_g);
      eg[tid] = e;
      bex[tid] = bv * e;
      dl[tid] = __expf(r_gl - r_g);
    }
    __syncthreads();
    const float eLc = __expf(gam[63]);
    // Output chunks have the longest per-chunk path: their next-chunk loads are
    // issued after the key pass (below) so their registers do not overlap the
    // P^T and (Q S)^T accumulators.
    if (!OUT && c + 1 < sr.c1) prefetch(c + 1);

    // chunk-start state out.  Value-major ([V][K]): a lane's four consecutive
    // keys of one value column are 8 contiguous bytes, stored straight from
    // registers.  Key-major ([K][V]): staged in LDS for 16-byte row stores.
    if (HOUT) {
      if (MODE == MODE_STATE || a.h_vm) {
        // packed: one 16-byte operand fragment per lane and block
        const __amdgpu_buffer_rsrc_t hrs =
            buf_rsrc(reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) {
            const typename VT<T>::x8 f = pack_split<T>(S[2 * kb2][vb], S[2 * kb2 + 1][vb]);
            buf_store16(hrs, packed_off((cb0 + cw0) / 16 + vb, kb2, l) * (int)sizeof(T),
                        __builtin_bit_cast(uint4, f));
          }
      } else if (a.h_svf) {
        const __amdgpu_buffer_rsrc_t hrs =
            buf_rsrc(reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) {
            const int vc = cb0 + cw0 + 16 * vb + col;
            const typename VT<T>::x4 hv{from_f<T>(S[kb][vb][0]), from_f<T>(S[kb][vb][1]),
                                        from_f<T>(S[kb][vb][2]), from_f<T>(S[kb][vb][3])};
            buf_store8(hrs, (vc * kDim + 16 * kb + 4 * grp) * (int)sizeof(T), __builtin_bit_cast(u32x2, hv));
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int vb = 0; vb < VB; ++vb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = 16 * kb + 4 * grp + e, lc = cw0 + 16 * vb + col;
              Hs[key * (CW + 8) + lc] = from_f<T>(S[kb][vb][e]);
            }
      }
    }

    // One pass over the key dimension forms, from the same K and Q fragments:
    //   K S            (B operand: S, register-local)
    //   (Q S)^T = S^T Q^T   (A operand: the same S registers; B: Q fragments)
    //   P^T = K Q^T    (upper-triangular 16x16 tiles (ib <= rb), in registers)
    x8 Sb[4][VB];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) Sb[kb2][vb] = pack_split<T>(S[2 * kb2][vb], S[2 * kb2 + 1][vb]);
    f32x4 ks[4][VB], qsT[VB][4], pT[10];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        ks[tb][vb] = zero4();
        qsT[vb][tb] = zero4();
      }
#pragma unroll
    for (int x = 0; x < 10; ++x) pT[x] = zero4();
    // The scheduling barrier closes each key block: hoisting the next block's
    // fragment reads above it would spill at two workgroups per CU.
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      x8 fk[4], fq[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) fk[tb] = frag_row_split(Ks + 16 * tb * LD + 32 * kb2, LD);
      if (OUT) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) fq[tb] = frag_row_split(Qs + 16 * tb * LD + 32 * kb2, LD);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) ks[tb][vb] = mfma16(fk[tb], Sb[kb2][vb], ks[tb][vb]);
      if (OUT) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
          for (int vb = 0; vb < VB; ++vb) qsT[vb][rb] = mfma16(Sb[kb2][vb], fq[rb], qsT[vb][rb]);
#pragma unroll
          for (int ib = 0; ib <= rb; ++ib) pT[tri_idx(ib, rb)] = mfma16(fk[ib], fq[rb], pT[tri_idx(ib, rb)]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (OUT && c + 1 < sr.c1) prefetch(c + 1);
    if (HST && !a.h_vm && !a.h_svf) {
      __syncthreads();  // every wave's part of the staged state is in Hs
      T* hp = reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV;
      constexpr int PR = CW / 8;
      for (int x = tid; x < 128 * PR; x += 256) {
        const int r = x / PR, c8 = (x % PR) * 8;
        *reinterpret_cast<uint4*>(hp + (int64_t)r * kDim + cb0 + c8) =
            *reinterpret_cast<const uint4*>(Hs + r * (CW + 8) + c8);
      }
    }

    // R = diag(beta) V - diag(beta e^gamma) K S   (in place in ks)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const f32x4 bt = *reinterpret_cast<const f32x4*>(bet + 16 * tb + 4 * grp);
      const f32x4 bx = *reinterpret_cast<const f32x4*>(bex + 16 * tb + 4 * grp);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        const f32x4 vd = isT ? zero4() : frag_d4(Vs, LDV, 16 * tb, cw0 + 16 * vb);
#pragma unroll
        for (int e = 0; e < 4; ++e) ks[tb][vb][e] = bt[e] * vd[e] - bx[e] * ks[tb][vb][e];
      }
    }
    // Delta = A R (A lower triangular: token block kb <= tb / 2)
    x8 Rb[2][VB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) Rb[kb][vb] = pack_split<T>(ks[2 * kb][vb], ks[2 * kb + 1][vb]);
    f32x4 dd[4][VB];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      x8 fa[2];
#pragma unroll
      for (int kb = 0; kb <= tb / 2; ++kb) fa[kb] = frag_row_split(As + 16 * tb * LDA + 32 * kb, LDA);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb <= tb / 2; ++kb) acc = mfma16(fa[kb], Rb[kb][vb], acc);
        dd[tb][vb] = acc;
      }
    }
    if (OUT) {
      // P^T[i][r] = (k_i . q_r) e^{gamma_r - gamma_i} for i <= r: tile (ib, rb)
      // holds rows i = 16 ib + 4 grp + e, column r = 16 rb + col
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float gr = gam[16 * rb + col];
#pragma unroll
        for (int ib = 0; ib <= rb; ++ib) {
          const f32x4 gi = *reinterpret_cast<const f32x4*>(gam + 16 * ib + 4 * grp);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // masked entries take exp(-inf) = 0: a select on the argument keeps
            // the exponential unconditional (a conditional one becomes a branch)
            const bool keep = (ib < rb) || (4 * grp + e <= col);
            pT[tri_idx(ib, rb)][e] *= __expf(keep ? gr - gi[e] : -INFINITY);
          }
        }
      }
      // O^T = diag-columns(e^gamma) (Q S)^T + Delta^T P^T; the A operand Delta^T
      // is the Delta accumulators themselves
      x8 Db[2][VB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) Db[kb][vb] = pack_split<T>(dd[2 * kb][vb], dd[2 * kb + 1][vb]);
      const int ors_ld = a.Hv * kDim * (int)sizeof(T);
      const __amdgpu_buffer_rsrc_t ors =
          buf_rsrc(reinterpret_cast<T*>(a.o) + (t0 * a.Hv + h) * kDim + vcol0, (int64_t)Cc * ors_ld);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const float er = eg[16 * rb + col];
        x8 pb[2];
#pragma unroll
        for (int kb = 0; kb <= rb / 2; ++kb)
          pb[kb] = pack_split<T>(pT[tri_idx(2 * kb, rb)],
                                 (2 * kb + 1 <= rb) ? pT[tri_idx(2 * kb + 1 < 4 ? 2 * kb + 1 : 3, rb)] : zero4());
        const int r = 16 * rb + col;
#pragma unroll
        for (int vb = 0; vb < VB; ++vb) {
          f32x4 acc = qsT[vb][rb] * er;
#pragma unroll
          for (int kb = 0; kb <= rb / 2; ++kb) acc = mfma16(Db[kb][vb], pb[kb], acc);
          acc *= a.scale;
          const typename VT<T>::x4 ov{from_f<T>(acc[0]), from_f<T>(acc[1]), from_f<T>(acc[2]),
                                      from_f<T>(acc[3])};
          // rows past the chunk's end fall outside the buffer range: dropped
          buf_store8(ors, r * ors_ld + (cw0 + 16 * vb + 4 * grp) * (int)sizeof(T),
                     __builtin_bit_cast(u32x2, ov));
        }
      }
    }
    // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta
    x8 Eb[2][VB];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(dl + 32 * kt + 4 * grp);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(dl + 32 * kt + 16 + 4 * grp);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) Eb[kt][vb] = pack_split<T>(dd[2 * kt][vb] * d0, dd[2 * kt + 1][vb] * d1);
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      x8 fk[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) fk[kt] = frag_tr_split(Ks + 32 * kt * LD + 16 * kb, LD);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        f32x4 acc = S[kb][vb] * eLc;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) acc = mfma16(fk[kt], Eb[kt][vb], acc);
        S[kb][vb] = acc;
      }
    }
  }

  if (MODE == MODE_AUG) {
    // T_seg to the kept transitions when there are any, else beside B_seg
    const bool kept = isT && a.trans;
    float* so = kept ? a.trans + ((int64_t)unit * a.P + p) * KV
                     : a.seg_out + ((int64_t)unit * a.P + p) * (2 * KV);
    const int ld = kept ? kDim : 2 * kDim;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, lc = cw0 + 16 * vb + col;
          so[key * ld + cb0 + lc] = S[kb][vb][e];
        }
  } else if (a.ht && p == sr.p_last) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < VB; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = vcol0 + cw0 + 16 * vb + col;
          a.ht[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = S[kb][vb][e];
        }
  }
}

template <typename T, int VB, int MODE>
__global__ __launch_bounds__(256, (VB == 1 && (MODE == MODE_AUG || MODE == MODE_STATE)) ? 2 : 1) void scan_kernel(ScanArgs a) {
  scan_body<T, VB, MODE>(a, (int)blockIdx.x, (int)gridDim.x);
}

// Forward output pass with specialized waves (one 64-column block per
// workgroup, 8 waves).  Waves 0-3 run the state chain of chunk c -- K S, R,
// Delta, the state update; waves 4-7 form the output of chunk c-1 from what
// the state waves left in LDS (the chunk-start state and Delta as MFMA
// operand registers, copied lane for lane) and the P tiles they computed
// themselves one iteration earlier, then the P tiles of chunk c.
// The output work is thus off the state chain's critical path, and two waves
// share each SIMD.  Chunk tiles are double-buffered where both roles read
// them (q, k, P, e^gamma, the operand copies).
//
// MODE_STATE (the backward's chunk-start states) uses the same split with
// waves 4-7 only loading and storing the chunk tiles, and the state waves
// writing h (packed) straight from registers; the output pass writes packed h
// from the operand copies when asked for it.  OPT (template flags, so
// the default path carries none of their code): bit 0 normalises the q / k
// rows after their loads, bit 1 maps beta through the runtime beta options.
template <typename T, int MODE, int OPT, int NCW = 4>
__device__ __forceinline__ void scan_spec_body(const ScanArgs& a, int b, int nb) {
  typedef typename VT<T>::x8 x8;
  constexpr bool OUT = (MODE == MODE_OUT);
  static_assert(NCW == 4 || (NCW == 2 && OUT), "two state waves only for the output pass");
  constexpr int CW = 16 * NCW;     // value columns per workgroup
  constexpr int NVS = 128 / CW;    // column blocks per (unit, segment)
  constexpr int NB = OUT ? 2 : 1;  // buffers of the tiles both roles read
  constexpr int LDV = CW + 8;      // v tile
  constexpr int LDA = 72;   // A and P tiles
  __shared__ __align__(16) T Qs[NB][OUT ? QK_TILE : 8];  // staggered rows (qk_row)
  __shared__ __align__(16) T Ks[NB][QK_TILE];
  __shared__ __align__(16) T Vs[64 * LDV];
  __shared__ __align__(16) T As[64 * LDA];
  __shared__ __align__(16) T Ps[NB][OUT ? 64 * LDA : 8];
  __shared__ __align__(16) x8 Xs[NB][NCW][4][OUT ? 64 : 1];  // S_c operands: [buf][column block][k block][lane]
  __shared__ __align__(16) x8 Xd[NB][NCW][2][OUT ? 64 : 1];  // Delta_c operands
  __shared__ __align__(16) float gam[64], bet[64], bex[64], dl[64], eg[2][64];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const bool outw = w >= NCW;
  // state waves: their 16-column block; output waves: their index 0..3
  const int wq = NCW == 4 ? (w & 3) : (outw ? w - NCW : w);
  const BlockPos bp = block_pos(a.order, b, nb, a.P * NVS, a.Hv);
  const int vs = bp.sub % NVS;
  const int p = bp.sub / NVS, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const SegRange sr = seg_range(nch, a.P, p);
  if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;  // empty segment
  const int cb0 = CW * vs;
  const int cw0 = (NCW == 4 || !outw) ? 16 * wq : 0;
  const int64_t KV = (int64_t)kDim * kDim;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  const T* Ag = reinterpret_cast<const T*>(a.A);
  const T* beta = reinterpret_cast<const T*>(a.beta);

  // initial state, every load issued before the first is used (a null source
  // reads zeros); the source is block-uniform, so the output waves load it
  // too (and never use it)
  f32x4 S[8];
  {
    const float* src = (p == 0) ? (a.h0 ? a.h0 + unit * KV : nullptr)
                                : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == 0) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw0 + col;
        S[kb][e] = buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
      }
  }

  // register prefetch of one chunk by the output waves (256 threads): the
  // vector-memory issue of a chunk's tiles takes hundreds of cycles, which
  // the state chain does not wait for
  const int otid = tid - 64 * NCW;
  TileRegs<128, 256> rq, rk;
  TileRegs<CW, 256> rv;
  TileRegs<64, 256> ra;
  float r_g = 0.f, r_gl = 0.f;
  T r_b = from_f<T>(0.f);
  bool r_ok = false;  // the row is inside the chunk
  auto prefetch = [&](int c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    if (OUT) tile_load<T, 128, 256>(rq, q + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, otid);
    tile_load<T, 128, 256>(rk, k + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, otid);
    tile_load<T, CW, 256>(rv, v + (t0 * a.Hv + h) * kDim + cb0, (int64_t)a.Hv * kDim, Cc, otid);
    tile_load<T, 64, 256>(ra, Ag + (t0 * a.Hv + h) * kChunk, (int64_t)a.Hv * kChunk, Cc, otid);
    if (otid < 64) {
      r_g = a.gcum[(t0 + min(otid, Cc - 1)) * a.Hv + h];
      r_gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
      r_b = (otid < Cc) ? beta[(t0 + otid) * a.Hv + h] : from_f<T>(0.f);
      r_ok = otid < Cc;
    }
  };

  // The initial state has arrived before the loop starts: otherwise the
  // compiler, merging the loop entry with the back edge, waits for every
  // outstanding load (the prefetch included) before the first use of S.
  __builtin_amdgcn_s_waitcnt(0);
  if (OUT) {
    p_zero_tiles<T>(Ps[0], LDA);
    p_zero_tiles<T>(Ps[NB - 1], LDA);
  }
  if (outw && sr.c0 < sr.c1) prefetch(sr.c0);
  // iteration it: state chain of chunk it (it < c1), output of chunk it-1
  // (it > c0); the last iteration only drains the output
  for (int it = sr.c0; it < sr.c1 + (OUT ? 1 : 0); ++it) {
    const int b = OUT ? (it & 1) : 0;
    __syncthreads();  // iteration it-1 is done with every buffer rewritten here
    if (outw && it < sr.c1) {
      if (OPT & 1) {
        if (OUT) l2norm_rows<T, 256>(rq, nullptr, otid);
        l2norm_rows<T, 256>(rk, nullptr, otid);
      }
      if (OUT) tile_store_q<T, 256>(Qs[b], rq, otid);
      tile_store_q<T, 256>(Ks[b], rk, otid);
      tile_store<T, CW, 256>(Vs, LDV, rv, otid);
      tile_store<T, 64, 256>(As, LDA, ra, otid);
      if (otid < 64) {
        const float bv = (OPT & 2) ? (r_ok ? beta_used(to_f(r_b), a.beta_mode) : 0.f) : to_f(r_b);
        const float e = __expf(r_g);
        gam[otid] = r_g;
        bet[otid] = bv;
        eg[b][otid] = e;
        bex[otid] = bv * e;
        dl[otid] = __expf(r_gl - r_g);
      }
    }
    __syncthreads();
    if (OUT && outw && a.h != nullptr && it > sr.c0) {
      // chunk-start state of chunk it-1 out, packed (the output pass writes
      // h only in that layout), from the state waves' operand copy.  Issued
      // before the prefetch, so the wait for the prefetched tiles does not
      // also wait for these stores.
      const int c = it - 1, bo = c & 1;
      constexpr int KPW = 4 * NCW / 4;  // k blocks per output wave
      const int cbk = wq % NCW;
      const __amdgpu_buffer_rsrc_t hrs = buf_rsrc(
          reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const int kb2 = (wq / NCW) * KPW + j;
        buf_store16(hrs, packed_off(cb0 / 16 + cbk, kb2, l) * (int)sizeof(T),
                    __builtin_bit_cast(uint4, Xs[bo][cbk][kb2][l]));
      }
    }
    if (outw && it + 1 < sr.c1) prefetch(it + 1);

    if (!outw) {
      if (it < sr.c1) {
        const float eLc = __expf(gam[63]);
        x8 Sb[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
          Sb[kb2] = pack_split<T>(S[2 * kb2], S[2 * kb2 + 1]);
          if (OUT) Xs[b][wq][kb2][l] = Sb[kb2];
        }
        if (MODE == MODE_STATE) {
          // chunk-start state out, packed: the operand fragments just formed
          const __amdgpu_buffer_rsrc_t hrs = buf_rsrc(
              reinterpret_cast<T*>(a.h) + ((choff + it) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
          for (int kb2 = 0; kb2 < 4; ++kb2)
            buf_store16(hrs, packed_off((cb0 + cw0) / 16, kb2, l) * (int)sizeof(T),
                        __builtin_bit_cast(uint4, Sb[kb2]));
        }
        // K S
        f32x4 ks[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) ks[tb] = zero4();
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            ks[tb] = mfma16(frag_row_split_q(Ks[b], 16 * tb, 32 * kb2), Sb[kb2], ks[tb]);
        // R = diag(beta) V - diag(beta e^gamma) K S
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(bet + 16 * tb + 4 * grp);
          const f32x4 bx = *reinterpret_cast<const f32x4*>(bex + 16 * tb + 4 * grp);
          const f32x4 vd = frag_d4(Vs, LDV, 16 * tb, cw0);
#pragma unroll
          for (int e = 0; e < 4; ++e) ks[tb][e] = bt[e] * vd[e] - bx[e] * ks[tb][e];
        }
        // Delta = A R
        const x8 Rb0 = pack_split<T>(ks[0], ks[1]), Rb1 = pack_split<T>(ks[2], ks[3]);
        f32x4 dd[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          f32x4 acc = mfma16(frag_row_split(As + 16 * tb * LDA, LDA), Rb0, zero4());
          if (tb >= 2) acc = mfma16(frag_row_split(As + 16 * tb * LDA + 32, LDA), Rb1, acc);
          dd[tb] = acc;
        }
        if (OUT) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) Xd[b][wq][kb][l] = pack_split<T>(dd[2 * kb], dd[2 * kb + 1]);
        }
        // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta
        x8 Eb[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(dl + 32 * kt + 4 * grp);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(dl + 32 * kt + 16 + 4 * grp);
          Eb[kt] = pack_split<T>(dd[2 * kt] * d0, dd[2 * kt + 1] * d1);
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          f32x4 acc = S[kb] * eLc;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) acc = mfma16(frag_tr_split_q(Ks[b], 32 * kt, 16 * kb), Eb[kt], acc);
          S[kb] = acc;
        }
      }
    } else if (OUT) {
      if (it > sr.c0) {
      // output of chunk c = it - 1:
      //   O^T = (Q S)^T diag(e^gamma) + Delta^T P^T, times scale
      // for column block cbk, row blocks rb0 .. rb0 + NCW - 1
      const int c = it - 1, bo = c & 1;
      const int cbk = wq % NCW, rb0 = (wq / NCW) * NCW;
      const int64_t t0 = s.start + (int64_t)kChunk * c;
      const int Cc = (int)min((int64_t)kChunk, s.end - t0);
      f32x4 qsT[NCW];
#pragma unroll
      for (int i = 0; i < NCW; ++i) qsT[i] = zero4();
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const x8 sb = Xs[bo][cbk][kb2][l];
#pragma unroll
        for (int i = 0; i < NCW; ++i)
          qsT[i] = mfma16(sb, frag_row_split_q(Qs[bo], 16 * (rb0 + i), 32 * kb2), qsT[i]);
      }
      const x8 Db0 = Xd[bo][cbk][0][l], Db1 = Xd[bo][cbk][1][l];
      const int ld_o = a.Hv * kDim * (int)sizeof(T);
      const __amdgpu_buffer_rsrc_t ors =
          buf_rsrc(reinterpret_cast<T*>(a.o) + (t0 * a.Hv + h) * kDim + cb0, (int64_t)Cc * ld_o);
#pragma unroll
      for (int i = 0; i < NCW; ++i) {
        const int rb = rb0 + i;
        f32x4 acc = qsT[i] * eg[bo][16 * rb + col];
        acc = mfma16(Db0, frag_row_split(Ps[bo] + 16 * rb * LDA, LDA), acc);
        if (rb >= 2) acc = mfma16(Db1, frag_row_split(Ps[bo] + 16 * rb * LDA + 32, LDA), acc);
        acc *= a.scale;
        const typename VT<T>::x4 ov{from_f<T>(acc[0]), from_f<T>(acc[1]), from_f<T>(acc[2]),
                                    from_f<T>(acc[3])};
        // rows past the chunk's end fall outside the buffer range: dropped
        buf_store8(ors, (16 * rb + col) * ld_o + (16 * cbk + 4 * grp) * (int)sizeof(T),
                   __builtin_bit_cast(u32x2, ov));
      }
      }
      // P of chunk it for the next iteration (tiles spread over the four waves)
      if (it < sr.c1) p_tiles<T, LAY_STAG>(Qs[b], Ks[b], 128, Ps[b], LDA, gam, wq);
    }
  }

  if (OUT && !outw && a.ht && p == sr.p_last) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + cw0 + col;
        a.ht[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = S[kb][e];
      }
  }
}

template <typename T, int OPT, int NCW>
__global__ __launch_bounds__(64 * (NCW + 4)) void scan_out_kernel(ScanArgs a) {
  scan_spec_body<T, MODE_OUT, OPT, NCW>(a, (int)blockIdx.x, (int)gridDim.x);
}

// The 32-column output pass with a loader wave (8 waves).  Waves 0-1 run the
// state chain of chunk it (16 value columns each); waves 2, 3, 6, 7 write the
// chunk-start state and the output of chunk it-1, P included (each forms the
// P tiles of its own rows in registers, from the q fragments its (Q S)^T
// product reads anyway); wave 4 copies the tiles of chunk it+1 from HBM into
// LDS with LDS-direct loads (no registers, no LDS stores by the compute
// waves), waits for them and publishes the chunk's per-row values, all before
// the one barrier per chunk, so the copies have a whole chunk's time to land.
// Wave 5 has no work: waves are dealt to the SIMDs in turn (w % 4), and with
// it the state chains share their SIMDs with the loader and an idle wave
// only while the output waves pair up on the other two (7 waves, one state
// chain sharing with an output wave, was 5 us slower at B=2 T=4096 H=32;
// wave 5 storing h, 8 us).  Buffers: q, k, gamma and e^gamma three-deep (the
// output of it-1 and the state chain of it read two chunks while it+1
// arrives), v, A and the other row values two-deep.  The h and output stores
// are non-temporal (155 -> 151 us).  OPT bit 1 maps beta through the runtime
// beta options; q / k normalisation keeps scan_spec_body.
template <typename T, int OPT>
__device__ __forceinline__ void scan_out_ld_body(const ScanArgs& a, int b, int nb) {
  typedef typename VT<T>::x8 x8;
  static_assert((OPT & 1) == 0, "q / k normalisation runs in scan_spec_body");
  constexpr int CW = 32, NVS = 4;
  __shared__ __align__(16) T Qs[3][64 * 128];  // swizzled (sw_off)
  __shared__ __align__(16) T Ks[3][64 * 128];
  __shared__ __align__(16) T Vs[2][64 * CW];
  __shared__ __align__(16) T As[2][64 * 64];
  __shared__ __align__(16) x8 Xs[2][2][4][64];  // S_c operands: [buf][column block][k block][lane]
  __shared__ __align__(16) x8 Xd[2][2][2][64];  // Delta_c operands
  __shared__ __align__(16) float gam[3][64], eg[3][64], bet[2][64], bex[2][64], dl[2][64];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const BlockPos bp = block_pos(a.order, b, nb, a.P * NVS, a.Hv);
  const int vs = bp.sub % NVS;
  const int p = bp.sub / NVS, unit = bp.unit;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const SegRange sr = seg_range(nch, a.P, p);
  if (sr.c0 >= sr.c1 && !(nch == 0 && p == 0)) return;  // empty segment
  const int cb0 = CW * vs;
  const int64_t KV = (int64_t)kDim * kDim;
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;

  // the chunk's tiles into buffers c % 3 (q, k, gamma, e^gamma) and c % 2 (the rest)
  auto load_chunk = [&](int c) {
    const int bq = c % 3, bk = c & 1;
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    const int gq = a.Hq * kDim * (int)sizeof(T), gv = a.Hv * kDim * (int)sizeof(T),
              ga = a.Hv * kChunk * (int)sizeof(T);
    const float gr = a.gcum[(t0 + min(l, Cc - 1)) * a.Hv + h];
    const float gl = a.gcum[(t0 + Cc - 1) * a.Hv + h];
    const float br = to_f(reinterpret_cast<const T*>(a.beta)[(t0 + min(l, Cc - 1)) * a.Hv + h]);
    tile_dma<128>(buf_rsrc(reinterpret_cast<const T*>(a.q) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gq),
                  gq, Qs[bq]);
    tile_dma<128>(buf_rsrc(reinterpret_cast<const T*>(a.k) + (t0 * a.Hq + hq) * kDim, (int64_t)Cc * gq),
                  gq, Ks[bq]);
    tile_dma<CW>(buf_rsrc(reinterpret_cast<const T*>(a.v) + (t0 * a.Hv + h) * kDim + cb0,
                          (int64_t)Cc * gv),
                 gv, Vs[bk]);
    tile_dma<64>(buf_rsrc(reinterpret_cast<const T*>(a.A) + (t0 * a.Hv + h) * kChunk,
                          (int64_t)Cc * ga),
                 ga, As[bk]);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every copy has landed in LDS
    if (Cc < kChunk) {
      // rows past the chunk's end are zero whatever the copies left there
      const uint4 z = make_uint4(0, 0, 0, 0);
      for (int x = 16 * l; x < (kChunk - Cc) * 256; x += 1024) {
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Qs[bq]) + Cc * 256 + x) = z;
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Ks[bq]) + Cc * 256 + x) = z;
      }
      for (int x = 16 * l; x < (kChunk - Cc) * 2 * CW; x += 1024)
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Vs[bk]) + Cc * 2 * CW + x) = z;
      for (int x = 16 * l; x < (kChunk - Cc) * 128; x += 1024)
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(As[bk]) + Cc * 128 + x) = z;
    }
    const bool ok = l < Cc;
    const float bv = ok ? ((OPT & 2) ? beta_used(br, a.beta_mode) : br) : 0.f;
    const float e = __expf(gr);
    gam[bq][l] = gr;
    bet[bk][l] = bv;
    bex[bk][l] = bv * e;
    dl[bk][l] = __expf(gl - gr);
    eg[bq][l] = e;
  };

  f32x4 S[8];
  if (w < 2) {
    const float* src = (p == 0) ? (a.h0 ? a.h0 + unit * KV : nullptr)
                                : a.seg_start + ((int64_t)unit * a.P + p) * KV;
    const bool vf = (p == 0) && a.svf;
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(src, src ? KV * (int64_t)sizeof(float) : 0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + 16 * w + col;
        S[kb][e] = buf_load_f32(srs, (vf ? vc * kDim + key : key * kDim + vc) * (int)sizeof(float));
      }
  } else if (w == 4 && sr.c0 < sr.c1) {
    load_chunk(sr.c0);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // iteration it: state chain of chunk it (it < c1), output of chunk it-1
  // (it > c0), copies of chunk it+1; the last iteration only drains the output
  for (int it = sr.c0; it <= sr.c1; ++it) {
    __syncthreads();  // chunk it is in LDS; iteration it-1 is done with what it+1 overwrites
    const int b = it & 1, bq = it % 3;
    if (w == 4) {
      if (it + 1 < sr.c1) load_chunk(it + 1);
    } else if (w < 2) {
      if (it < sr.c1) {
        const int cw0 = 16 * w;
        const float eLc = __expf(gam[bq][63]);
        x8 Sb[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
          Sb[kb2] = pack_split<T>(S[2 * kb2], S[2 * kb2 + 1]);
          Xs[b][w][kb2][l] = Sb[kb2];
        }
        // K S
        f32x4 ks[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) ks[tb] = zero4();
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
            ks[tb] = mfma16(frag_row_split_w<T, 128>(Ks[bq], 16 * tb, 32 * kb2), Sb[kb2], ks[tb]);
        // R = diag(beta) V - diag(beta e^gamma) K S
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const f32x4 bt = *reinterpret_cast<const f32x4*>(bet[b] + 16 * tb + 4 * grp);
          const f32x4 bx = *reinterpret_cast<const f32x4*>(bex[b] + 16 * tb + 4 * grp);
          const f32x4 vd = frag_d4_w<T, CW>(Vs[b], 16 * tb, cw0);
#pragma unroll
          for (int e = 0; e < 4; ++e) ks[tb][e] = bt[e] * vd[e] - bx[e] * ks[tb][e];
        }
        // Delta = A R
        const x8 Rb0 = pack_split<T>(ks[0], ks[1]), Rb1 = pack_split<T>(ks[2], ks[3]);
        f32x4 dd[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          f32x4 acc = mfma16(frag_row_split_w<T, 64>(As[b], 16 * tb, 0), Rb0, zero4());
          if (tb >= 2) acc = mfma16(frag_row_split_w<T, 64>(As[b], 16 * tb, 32), Rb1, acc);
          dd[tb] = acc;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Xd[b][w][kb][l] = pack_split<T>(dd[2 * kb], dd[2 * kb + 1]);
        // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta
        x8 Eb[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(dl[b] + 32 * kt + 4 * grp);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(dl[b] + 32 * kt + 16 + 4 * grp);
          Eb[kt] = pack_split<T>(dd[2 * kt] * d0, dd[2 * kt + 1] * d1);
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          f32x4 acc = S[kb] * eLc;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            acc = mfma16(frag_tr_split_w<T, 128>(Ks[bq], 32 * kt, 16 * kb), Eb[kt], acc);
          S[kb] = acc;
        }
      }
    } else if (w != 5 && it > sr.c0) {
      // waves 2, 3, 6, 7 -> 0..3: value column block cbk, row blocks
      // {rA, rB} = {0, 3} or {1, 2} (equal shares of the triangular P)
      const int wq = (w & 1) | ((w >> 1) & 2), cbk = wq & 1;
      const int rA = wq >> 1, rB = 3 - rA;
      const int c = it - 1, bo = c & 1, bqo = (bq + 2) % 3;
      if (a.h != nullptr) {
        // chunk-start state of chunk c out, packed, from the operand copy
        const __amdgpu_buffer_rsrc_t hrs = buf_rsrc(
            reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV, KV * (int64_t)sizeof(T));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int kb2 = (wq >> 1) * 2 + j;
          buf_store16_nt(hrs, packed_off(cb0 / 16 + cbk, kb2, l) * (int)sizeof(T),
                      __builtin_bit_cast(uint4, Xs[bo][cbk][kb2][l]));
        }
      }
      // O^T = (Q S)^T diag(e^gamma) + Delta^T P^T, times scale, rows rA and rB.
      // The q fragments of both row blocks serve (Q S)^T and P^T = K Q^T, the
      // latter kept in registers: tiles (cb, rA) for cb < 2 and (cb, rB) for
      // all cb (those above the diagonal come out zero), each gated by
      // e^{gamma_t - gamma_i} on and below it.
      const T* Qc = Qs[bqo];
      const T* Kc = Ks[bqo];
      const float* gc = gam[bqo];
      x8 fq[2][4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        fq[0][kb2] = frag_row_split_w<T, 128>(Qc, 16 * rA, 32 * kb2);
        fq[1][kb2] = frag_row_split_w<T, 128>(Qc, 16 * rB, 32 * kb2);
      }
      f32x4 qsT[2] = {zero4(), zero4()};
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const x8 sb = Xs[bo][cbk][kb2][l];
        qsT[0] = mfma16(sb, fq[0][kb2], qsT[0]);
        qsT[1] = mfma16(sb, fq[1][kb2], qsT[1]);
      }
      f32x4 pa[2], pb[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        x8 fk[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) fk[kb2] = frag_row_split_w<T, 128>(Kc, 16 * cb, 32 * kb2);
        f32x4 accb = zero4();
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) accb = mfma16(fk[kb2], fq[1][kb2], accb);
        pb[cb] = accb;
        if (cb < 2) {
          f32x4 acca = zero4();
#pragma unroll
          for (int kb2 = 0; kb2 < 4; ++kb2) acca = mfma16(fk[kb2], fq[0][kb2], acca);
          pa[cb] = acca;
        }
      }
      // gate and mask: lane (grp, col) of tile (cb, r) holds P[t][i] with
      // t = 16 r + col, i = 16 cb + 4 grp + e; masked entries take exp(-inf)
      const float gtA = gc[16 * rA + col], gtB = gc[16 * rB + col];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const f32x4 gi = *reinterpret_cast<const f32x4*>(gc + 16 * cb + 4 * grp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * cb + 4 * grp + e;
          pb[cb][e] *= __expf(i <= 16 * rB + col ? gtB - gi[e] : -INFINITY);
          if (cb < 2) pa[cb][e] *= __expf(i <= 16 * rA + col ? gtA - gi[e] : -INFINITY);
        }
      }
      const x8 Db0 = Xd[bo][cbk][0][l], Db1 = Xd[bo][cbk][1][l];
      const int64_t t0 = s.start + (int64_t)kChunk * c;
      const int Cc = (int)min((int64_t)kChunk, s.end - t0);
      const int ld_o = a.Hv * kDim * (int)sizeof(T);
      const __amdgpu_buffer_rsrc_t ors =
          buf_rsrc(reinterpret_cast<T*>(a.o) + (t0 * a.Hv + h) * kDim + cb0, (int64_t)Cc * ld_o);
      f32x4 oA = qsT[0] * eg[bqo][16 * rA + col];
      oA = mfma16(Db0, pack_split<T>(pa[0], pa[1]), oA);  // rA < 2: keys 0..31 only
      f32x4 oB = qsT[1] * eg[bqo][16 * rB + col];
      oB = mfma16(Db0, pack_split<T>(pb[0], pb[1]), oB);
      oB = mfma16(Db1, pack_split<T>(pb[2], pb[3]), oB);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rb = i ? rB : rA;
        const f32x4 acc = (i ? oB : oA) * a.scale;
        const typename VT<T>::x4 ov{from_f<T>(acc[0]), from_f<T>(acc[1]), from_f<T>(acc[2]),
                                    from_f<T>(acc[3])};
        // rows past the chunk's end fall outside the buffer range: dropped
        buf_store8_nt(ors, (16 * rb + col) * ld_o + (16 * cbk + 4 * grp) * (int)sizeof(T),
                   __builtin_bit_cast(u32x2, ov));
      }
    }
  }

  if (w < 2 && a.ht && p == sr.p_last) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = cb0 + 16 * w + col;
        a.ht[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = S[kb][e];
      }
  }
}

template <typename T, int OPT>
__global__ __launch_bounds__(512) void scan_out_ld_kernel(ScanArgs a) {
  scan_out_ld_body<T, OPT>(a, (int)blockIdx.x, (int)gridDim.x);
}

// Pass 2: chain the segment start states of one (unit, 16-column block).
// Forward:  start[1] = B_0 (segment 0 ran from the initial state),
//           start[p] = T_{p-1} start[p-1] + B_{p-1},  p = 2 .. p_last.
// Reverse (state gradients, segments walked from the end): with G[p] the
// gradient entering segment p's end, G[p_last-1] = B_{p_last} (the last
// segment ran from dht), G[p] = T_{p+1} G[p+1] + B_{p+1}, p = p_last-2 .. 0.
// fp32 MFMA (16x16x4); wave w owns rows 32w .. 32w+31.
static __global__ __launch_bounds__(256) void cp_combine_kernel(ScanArgs a) {
  __shared__ float Sp[128 * 17];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const int unit = blockIdx.x >> 3, cblk = blockIdx.x & 7;
  const int n = unit / a.Hv;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const SegRange sr = seg_range(nch, a.P, 0);
  const int64_t KV = (int64_t)kDim * kDim;
  const int c0 = 16 * cblk;
  for (int jstep = 1; jstep <= sr.p_last; ++jstep) {
    const int p = a.reverse ? sr.p_last - jstep : jstep;
    const int src = a.reverse ? p + 1 : p - 1;
    const float* prev = a.seg_out + ((int64_t)unit * a.P + src) * (2 * KV);
    float* dst = const_cast<float*>(a.seg_start) + ((int64_t)unit * a.P + p) * KV;
    // the matrix applied to the chained value, element (r, s) at
    // tm[r * trs + s * tcs]: the transition beside B_seg in seg_out (the
    // backward's own pass 1 leaves the transposed one there), or the kept
    // forward transition, transposed for the backward
    const float* tm = a.trans ? a.trans + ((int64_t)unit * a.P + src) * KV : prev;
    const int trs = a.trans ? (a.reverse ? 1 : kDim) : 2 * kDim;
    const int tcs = (a.trans && a.reverse) ? kDim : 1;
    f32x4 acc[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r0 = 32 * w + 16 * rt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc[rt][e] = prev[(r0 + 4 * grp + e) * (2 * kDim) + kDim + c0 + col];
      if (jstep > 1) {
        for (int st = 0; st < 32; ++st) {
          const float av = tm[(r0 + col) * trs + (4 * st + grp) * tcs];
          const float bv = Sp[(4 * st + grp) * 17 + col];
          acc[rt] = mfma16f32(av, bv, acc[rt]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(r0 + 4 * grp + e) * kDim + c0 + col] = acc[rt][e];
    }
    __syncthreads();  // every wave is done reading the previous start state
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Sp[(32 * w + 16 * rt + 4 * grp + e) * 17 + col] = acc[rt][e];
    __syncthreads();
  }
}

}  // namespace gdr
