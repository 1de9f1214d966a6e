// gdr_fwd.hip -- forward kernels of the chunked gated delta rule on gfx950.
//
// The forward of the FlashQLA pages ("flashqla-linear-attention", Low-Level
// API; "FlashQLA Documentation", forward pass: g, A, o, h, final_state) in two
// launches:
//
//   fwd_prep  one workgroup per (chunk, value head), fully parallel:
//             gamma = chunk-local inclusive cumsum of g            -> g_cum
//             M = strict_lower(diag(beta) K K^T o exp(gamma_r - gamma_i))
//             A = (I + M)^{-1}, unit lower triangular (fp32, blocked:
//             16x16 diagonal blocks by substitution, off-diagonal blocks by
//             fp32 MFMA)                                            -> A
//   fwd_scan  one workgroup per (sequence, value head), sequential over the
//             sequence's chunks; wave w owns value columns [32w, 32w+32) of
//             the 128 x 128 fp32 state S, held in MFMA accumulators:
//             R = diag(beta) V - diag(beta e^gamma) (K S)
//             Delta = A R                   (= U - W S of the WY form)
//             O = scale (diag(e^gamma) Q S + lower_incl(Q K^T o Gamma) Delta)
//             S <- e^{gamma_L} S + K^T (diag(e^{gamma_L - gamma}) Delta)
//
// Every contraction is a 16x16x32 bf16/fp16 MFMA with fp32 accumulation;
// S and R, Delta enter the next product as register-local B operands.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* h0;
  float* gcum;
  void* A;
  void* o;
  void* h;
  float* ht;
  const int32_t* cu;    // device cu_seqlens, or null for dense batches
  const int32_t* offs;  // device chunk offsets [N+1] (packed input only)
  int N, T, Hq, Hv;
  int nc_dense;
  int g_dtype;
  float scale;
  int svf;
};

// Chunk offsets of packed sequences, computed on the device so that no
// device-to-host copy is needed: offs[0] = 0, offs[n+1] = offs[n] +
// ceil(len_n / 64).
__global__ void chunk_offsets_kernel(const int32_t* cu, int N, int32_t* offs) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int32_t acc = 0;
    offs[0] = 0;
    for (int n = 0; n < N; ++n) {
      acc += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
      offs[n + 1] = acc;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void fwd_prep_kernel(FwdArgs a) {
  constexpr int LDK = 136;
  constexpr int LDM = 68;
  __shared__ __align__(16) T Ks[64 * LDK];
  __shared__ float Mf[64 * LDM];
  __shared__ float Ai[64 * LDM];
  __shared__ float gam[64], bet[64];

  const int c = blockIdx.x, h = blockIdx.y;
  int n, j;
  if (a.cu) {
    n = find_seq(a.offs, a.N, c);
    j = c - a.offs[n];
  } else {
    n = c / a.nc_dense;
    j = c % a.nc_dense;
  }
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int64_t t0 = s.start + (int64_t)kChunk * j;
  const int Cc = (int)min((int64_t)kChunk, s.end - t0);
  const int G = a.Hv / a.Hq, hq = h / G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;

  if (w == 0) {
    const float gv = (l < Cc) ? load_scalar(a.g, (t0 + l) * a.Hv + h, a.g_dtype) : 0.f;
    const float gc = wave_inclusive_scan(gv);
    gam[l] = gc;
    bet[l] = (l < Cc) ? to_f(reinterpret_cast<const T*>(a.beta)[(t0 + l) * a.Hv + h]) : 0.f;
    if (l < Cc) a.gcum[(t0 + l) * a.Hv + h] = gc;
  }
  tile_to_lds<T, 256>(Ks, LDK, reinterpret_cast<const T*>(a.k) + (t0 * a.Hq + hq) * kDim,
                      (int64_t)a.Hq * kDim, Cc, kDim);
  __syncthreads();

  // M, rows 16w .. 16w+15 (only the blocks on or below the diagonal are nonzero)
  for (int cb = 0; cb < 4; ++cb) {
    f32x4 acc = zero4();
    if (cb <= w) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mfma16(frag_row(Ks + 16 * w * LDK + 32 * kk, LDK),
                     frag_row(Ks + 16 * cb * LDK + 32 * kk, LDK), acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * w + 4 * grp + e, i = 16 * cb + col;
      float m = 0.f;
      if (i < r) m = bet[r] * __expf(gam[r] - gam[i]) * acc[e];
      Mf[r * LDM + i] = m;
    }
  }
  // blocks above the diagonal of the inverse are zero
  for (int x = tid; x < 64 * 64; x += 256) {
    const int r = x >> 6, cc = x & 63;
    if ((cc >> 4) > (r >> 4)) Ai[r * LDM + cc] = 0.f;
  }
  __syncthreads();

  // diagonal 16x16 blocks: forward substitution, lane l < 16 owns column l
  if (l < 16) {
    const int b0 = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == l) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= Mf[(b0 + r) * LDM + b0 + i] * x[i];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ai[(b0 + r) * LDM + b0 + l] = x[r];
  }
  __syncthreads();

  // off-diagonal blocks by distance d from the diagonal:
  //   A_ij = -A_ii * sum_{j <= m < i} M_im A_mj
  for (int d = 1; d < 4; ++d) {
    if (w < 4 - d) {
      const int bi = w + d, bj = w;
      f32x4 t = zero4();
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float av = Mf[(16 * bi + col) * LDM + 16 * m + 4 * st + grp];
          const float bv = Ai[(16 * m + 4 * st + grp) * LDM + 16 * bj + col];
          t = mfma16f32(av, bv, t);
        }
      }
      // t is a D tile: lane (grp, col) holds t[4 grp + e][col]; step e of the
      // next product uses k = 4 grp + e for lane group grp.
      f32x4 r = zero4();
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float av = Ai[(16 * bi + col) * LDM + 16 * bi + 4 * grp + e];
        r = mfma16f32(av, t[e], r);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ai[(16 * bi + 4 * grp + e) * LDM + 16 * bj + col] = -r[e];
    }
    __syncthreads();
  }

  // A rows of the chunk, 8 elements (16 bytes) per store
  T* Aout = reinterpret_cast<T*>(a.A);
  for (int x = tid; x < 64 * 8; x += 256) {
    const int r = x >> 3, c8 = (x & 7) * 8;
    if (r < Cc) {
      typename VT<T>::x8 vals;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = c8 + e;
        vals[e] = from_f<T>(cc <= r ? Ai[r * LDM + cc] : 0.f);
      }
      *reinterpret_cast<typename VT<T>::x8*>(Aout + ((t0 + r) * a.Hv + h) * kChunk + c8) = vals;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void fwd_scan_kernel(FwdArgs a) {
  typedef typename VT<T>::x8 x8;
  constexpr int LD = 136;
  constexpr int LDA = 72;
  __shared__ __align__(16) T Qs[64 * LD];
  __shared__ __align__(16) T Ks[64 * LD];
  __shared__ __align__(16) T Vs[64 * LD];
  __shared__ __align__(16) T As[64 * LDA];
  __shared__ __align__(16) T Ps[64 * LDA];
  __shared__ float gam[64], bet[64], eg[64], bex[64], dl[64];

  const int unit = blockIdx.x;
  const int n = unit / a.Hv, h = unit % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, grp = l >> 4, col = l & 15;
  const SeqInfo s = seq_info(a.cu, n, a.T);
  const int nch = (int)((s.end - s.start + kChunk - 1) / kChunk);
  const int64_t choff = a.cu ? (int64_t)a.offs[n] : (int64_t)n * a.nc_dense;
  const int64_t KV = (int64_t)kDim * kDim;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* k = reinterpret_cast<const T*>(a.k);
  const T* v = reinterpret_cast<const T*>(a.v);
  const T* A = reinterpret_cast<const T*>(a.A);
  const T* beta = reinterpret_cast<const T*>(a.beta);
  T* o = reinterpret_cast<T*>(a.o);

  // state S[key][vcol]: tile (kb, vb) = keys 16kb.., columns 32w + 16vb..
  f32x4 S[8][2];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 16 * kb + 4 * grp + e, vc = 32 * w + 16 * vb + col;
        float x = 0.f;
        if (a.h0) x = a.h0[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)];
        S[kb][vb][e] = x;
      }

  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = s.start + (int64_t)kChunk * c;
    const int Cc = (int)min((int64_t)kChunk, s.end - t0);
    if (a.h) {
      T* hp = reinterpret_cast<T*>(a.h) + ((choff + c) * a.Hv + h) * KV;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = 16 * kb + 4 * grp + e, vc = 32 * w + 16 * vb + col;
            hp[a.svf ? vc * kDim + key : key * kDim + vc] = from_f<T>(S[kb][vb][e]);
          }
    }
    __syncthreads();  // the previous chunk is done with LDS
    tile_to_lds<T, 256>(Qs, LD, q + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, kDim);
    tile_to_lds<T, 256>(Ks, LD, k + (t0 * a.Hq + hq) * kDim, (int64_t)a.Hq * kDim, Cc, kDim);
    tile_to_lds<T, 256>(Vs, LD, v + (t0 * a.Hv + h) * kDim, (int64_t)a.Hv * kDim, Cc, kDim);
    tile_to_lds<T, 256>(As, LDA, A + (t0 * a.Hv + h) * kChunk, (int64_t)a.Hv * kChunk, Cc, kChunk);
    if (tid < 64) {
      const int r = min(tid, Cc - 1);  // rows past the end repeat the last gamma
      gam[tid] = a.gcum[(t0 + r) * a.Hv + h];
      bet[tid] = (tid < Cc) ? to_f(beta[(t0 + tid) * a.Hv + h]) : 0.f;
    }
    __syncthreads();
    if (tid < 64) {
      const float gr = gam[tid];
      eg[tid] = __expf(gr);
      bex[tid] = bet[tid] * __expf(gr);
      dl[tid] = __expf(gam[63] - gr);
    }
    // P = lower_incl(Q K^T o Gamma), rows 16w .. 16w+15
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 acc = zero4();
      if (cb <= w) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc = mfma16(frag_row(Qs + 16 * w * LD + 32 * kk, LD),
                       frag_row(Ks + 16 * cb * LD + 32 * kk, LD), acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * grp + e, i = 16 * cb + col;
        float p = 0.f;
        if (i <= r) p = acc[e] * __expf(gam[r] - gam[i]);
        Ps[r * LDA + i] = from_f<T>(p);
      }
    }
    __syncthreads();
    const float eL = __expf(gam[63]);

    // K S and Q S for this wave's 32 columns
    x8 Sb[4][2];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) Sb[kb2][vb] = pack_split<T>(S[2 * kb2][vb], S[2 * kb2 + 1][vb]);
    f32x4 ks[4][2], qs[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        ks[tb][vb] = zero4();
        qs[tb][vb] = zero4();
      }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        const x8 fk = frag_row_split(Ks + 16 * tb * LD + 32 * kb2, LD);
        const x8 fq = frag_row_split(Qs + 16 * tb * LD + 32 * kb2, LD);
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
          ks[tb][vb] = mfma16(fk, Sb[kb2][vb], ks[tb][vb]);
          qs[tb][vb] = mfma16(fq, Sb[kb2][vb], qs[tb][vb]);
        }
      }
    // R = diag(beta) V - diag(beta e^gamma) K S   (in place in ks)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + 4 * grp + e, vc = 32 * w + 16 * vb + col;
          ks[tb][vb][e] = bet[r] * to_f(Vs[r * LD + vc]) - bex[r] * ks[tb][vb][e];
        }
    // Delta = A R (A lower triangular: token block kb <= tb / 2)
    x8 Rb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) Rb[kb][vb] = pack_split<T>(ks[2 * kb][vb], ks[2 * kb + 1][vb]);
    f32x4 dd[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb <= tb / 2; ++kb)
          acc = mfma16(frag_row_split(As + 16 * tb * LDA + 32 * kb, LDA), Rb[kb][vb], acc);
        dd[tb][vb] = acc;
      }
    // O = scale (diag(e^gamma) Q S + P Delta)
    x8 Db[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) Db[kb][vb] = pack_split<T>(dd[2 * kb][vb], dd[2 * kb + 1][vb]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb <= tb / 2; ++kb)
          acc = mfma16(frag_row_split(Ps + 16 * tb * LDA + 32 * kb, LDA), Db[kb][vb], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + 4 * grp + e, vc = 32 * w + 16 * vb + col;
          if (r < Cc)
            o[((t0 + r) * a.Hv + h) * kDim + vc] =
                from_f<T>(a.scale * (eg[r] * qs[tb][vb][e] + acc[e]));
        }
      }
    // S <- e^{gamma_L} S + K^T diag(e^{gamma_L - gamma}) Delta
    x8 Eb[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 top = dd[2 * kt][vb], bot = dd[2 * kt + 1][vb];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          top[e] *= dl[32 * kt + 4 * grp + e];
          bot[e] *= dl[32 * kt + 16 + 4 * grp + e];
        }
        Eb[kt][vb] = pack_split<T>(top, bot);
      }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        f32x4 acc = S[kb][vb] * eL;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          acc = mfma16(frag_tr_split(Ks + 32 * kt * LD + 16 * kb, LD), Eb[kt][vb], acc);
        S[kb][vb] = acc;
      }
  }

  if (a.ht) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = 16 * kb + 4 * grp + e, vc = 32 * w + 16 * vb + col;
          a.ht[unit * KV + (a.svf ? vc * kDim + key : key * kDim + vc)] = S[kb][vb][e];
        }
  }
}

size_t fwd_workspace_bytes(const gdr_problem* p, const Plan& pl) {
  size_t b = 0;
  if (p->cu_seqlens_dev) b += align256(sizeof(int32_t) * (size_t)(pl.N + 1));
  return b;
}

template <typename T>
static gdr_status launch_fwd_t(const gdr_problem* p, const Plan& pl, FwdArgs a, hipStream_t st) {
  if (pl.total_chunks > 0) {
    hipLaunchKernelGGL(fwd_prep_kernel<T>, dim3((unsigned)pl.total_chunks, p->Hv), dim3(256), 0,
                       st, a);
  }
  hipLaunchKernelGGL(fwd_scan_kernel<T>, dim3((unsigned)(pl.N * p->Hv)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("kernel launch failed: %s", hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

gdr_status launch_fwd(const gdr_problem* p, const Plan& pl, const void* q, const void* k,
                      const void* v, const void* g, const void* beta, const float* h0,
                      float* gcum, void* A, void* o, void* h, float* ht, void* ws,
                      hipStream_t st) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.h0 = h0;
  a.gcum = gcum;
  a.A = A;
  a.o = o;
  a.h = h;
  a.ht = ht;
  a.cu = p->cu_seqlens_dev;
  a.offs = nullptr;
  a.N = pl.N;
  a.T = p->T;
  a.Hq = p->Hq;
  a.Hv = p->Hv;
  a.nc_dense = pl.nc_dense;
  a.g_dtype = (int)p->g_dtype;
  a.scale = p->scale;
  a.svf = p->state_v_first ? 1 : 0;
  if (p->cu_seqlens_dev) {
    int32_t* offs = reinterpret_cast<int32_t*>(ws);
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(64), 0, st, p->cu_seqlens_dev, pl.N,
                       offs);
    a.offs = offs;
  }
  if (p->in_dtype == GDR_BF16) return launch_fwd_t<__bf16>(p, pl, a, st);
  return launch_fwd_t<_Float16>(p, pl, a, st);
}

}  // namespace gdr
