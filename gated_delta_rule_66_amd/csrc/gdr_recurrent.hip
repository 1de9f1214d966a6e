// gdr_recurrent.hip -- the gated delta rule token by token, for short inputs
// on gfx950: decode steps, a few speculative tokens, or a prefill continued
// from a cached state (the state-cached continuation the FlashQLA skill page
// lists).  The chunked path needs 64-token chunks to pay off; here a
// workgroup walks the tokens one at a time with the state on chip.
//
// One 256-thread workgroup per (sequence, value head) holds the 128 x 128
// fp32 state in registers, 64 values per thread, reads it once and writes it
// once (in place when final_state == initial_state).  Per token, with the
// state S before the token:
//   a = e^g (g from the gate input when the gate is on);  s_k = S^T k;  s_q = S^T q
//   u = beta (v - a s_k)
//   o = scale (a s_q + (k . q) u)       (= scale S_new^T q, expanded)
//   S <- a S + k u^T
// so one cross-thread reduction per token serves both products.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

struct RecArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* h0;  // nullable
  float* ht;        // nullable; may equal h0
  void* o;
  const int32_t* cu;  // device cu_seqlens, or null for dense batches
  int N, T, Hq, Hv, g_dtype, qk_norm;
  int beta_mode;  // bit 0 sigmoid of a beta logit, bit 1 twice beta
  float scale;
  const float* gate_A_log;    // non-null: g is the gate input (gate_log_decay)
  const float* gate_dt_bias;  // nullable
};

// Thread t owns 16 four-wide pieces of the state.  SVF = 0 (state [K][V]):
// keys 16 (t / 32) + r, r < 16, each with value columns 4 (t % 32) .. + 3.
// SVF = 1 (state [V][K]): value columns 16 (t / 32) + c, c < 16, each with
// keys 4 (t % 32) .. + 3.  Either way the 32 threads of a half wave read or
// write one contiguous 512-byte state row per access.
template <typename T, bool SVF>
__global__ __launch_bounds__(256) void recurrent_kernel(RecArgs a) {
  constexpr int LR = 128 + 4;  // padded rows of the partial sums
  __shared__ __align__(16) float qs[2][128], ks[2][128];  // token vectors, by token parity
  __shared__ __align__(16) float us[128];
  __shared__ __align__(16) float red_k[32 * LR], red_q[32 * LR];
  __shared__ float kq_s[2];

  const int n = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
  const int G = a.Hv / a.Hq, hq = h / G;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int lo = tid & 31, hi = tid >> 5;  // piece index within / across half waves
  const float gate_a = a.gate_A_log ? a.gate_A_log[h] : 0.f;
  const float gate_b = a.gate_dt_bias ? a.gate_dt_bias[h] : 0.f;
  int64_t t_begin, t_end;
  if (a.cu) {
    t_begin = a.cu[n];
    t_end = a.cu[n + 1];
  } else {
    t_begin = (int64_t)n * a.T;
    t_end = t_begin + a.T;
  }
  constexpr int64_t KV = 128 * 128;
  // row r of this thread's pieces: state element offset of its first value
  auto piece = [&](int r) -> int { return (16 * hi + r) * 128 + 4 * lo; };

  float4 S[16];
  if (a.h0) {
    const float* src = a.h0 + ((int64_t)n * a.Hv + h) * KV;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = *reinterpret_cast<const float4*>(src + piece(r));
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* kg = reinterpret_cast<const T*>(a.k);
  const T* vg = reinterpret_cast<const T*>(a.v);
  const T* bg = reinterpret_cast<const T*>(a.beta);
  // token values in registers (loaded one token ahead): wave 0 holds q, k
  // elements 2l, 2l + 1; threads 0..127 hold v_j; every thread g and beta
  uint32_t rq = 0, rk = 0;
  float rv = 0.f, rg = 0.f, rb = 0.f;
  auto load_token = [&](int64_t t) {
    if (w == 0) {
      rq = *reinterpret_cast<const uint32_t*>(qg + (t * a.Hq + hq) * 128 + 2 * l);
      rk = *reinterpret_cast<const uint32_t*>(kg + (t * a.Hq + hq) * 128 + 2 * l);
    }
    if (tid < 128) rv = to_f(vg[(t * a.Hv + h) * 128 + tid]);
    rg = load_scalar(a.g, t * a.Hv + h, a.g_dtype);
    if (a.gate_A_log) rg = gate_log_decay(rg, gate_a, gate_b);
    rb = beta_used(to_f(bg[t * a.Hv + h]), a.beta_mode);
  };
  if (t_begin < t_end) load_token(t_begin);

  for (int64_t t = t_begin; t < t_end; ++t) {
    const int par = (int)(t & 1);
    // stage q, k (normalised when asked) and k . q
    if (w == 0) {
      const T* qp = reinterpret_cast<const T*>(&rq);
      const T* kp = reinterpret_cast<const T*>(&rk);
      float q0 = to_f(qp[0]), q1 = to_f(qp[1]), k0 = to_f(kp[0]), k1 = to_f(kp[1]);
      if (a.qk_norm) {
        const float iq = rsqrtf(sum4g(sum16(q0 * q0 + q1 * q1)) + kQKNormEps);
        const float ik = rsqrtf(sum4g(sum16(k0 * k0 + k1 * k1)) + kQKNormEps);
        q0 *= iq;
        q1 *= iq;
        k0 *= ik;
        k1 *= ik;
      }
      const float kq = sum4g(sum16(k0 * q0 + k1 * q1));
      qs[par][2 * l] = q0;
      qs[par][2 * l + 1] = q1;
      ks[par][2 * l] = k0;
      ks[par][2 * l + 1] = k1;
      if (l == 0) kq_s[par] = kq;
    }
    const float av = __expf(rg), bv = rb, vv = rv;
    __syncthreads();
    if (t + 1 < t_end) load_token(t + 1);

    // partial S^T k and S^T q over this thread's keys
    if (!SVF) {
      float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = ks[par][16 * hi + r], qr = qs[par][16 * hi + r];
        pk.x += S[r].x * kr; pk.y += S[r].y * kr; pk.z += S[r].z * kr; pk.w += S[r].w * kr;
        pq.x += S[r].x * qr; pq.y += S[r].y * qr; pq.z += S[r].z * qr; pq.w += S[r].w * qr;
      }
      *reinterpret_cast<float4*>(red_k + hi * LR + 4 * lo) = pk;
      *reinterpret_cast<float4*>(red_q + hi * LR + 4 * lo) = pq;
    } else {
      const float4 k4 = *reinterpret_cast<const float4*>(&ks[par][4 * lo]);
      const float4 q4 = *reinterpret_cast<const float4*>(&qs[par][4 * lo]);
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        float4 pk, pq;
        float* pkp = reinterpret_cast<float*>(&pk);
        float* pqp = reinterpret_cast<float*>(&pq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float4 s = S[4 * c4 + e];
          pkp[e] = s.x * k4.x + s.y * k4.y + s.z * k4.z + s.w * k4.w;
          pqp[e] = s.x * q4.x + s.y * q4.y + s.z * q4.z + s.w * q4.w;
        }
        *reinterpret_cast<float4*>(red_k + lo * LR + 16 * hi + 4 * c4) = pk;
        *reinterpret_cast<float4*>(red_q + lo * LR + 16 * hi + 4 * c4) = pq;
      }
    }
    __syncthreads();

    // column j = tid: the sums over key slots (fixed order), u and the output
    if (tid < 128) {
      constexpr int NS = SVF ? 32 : 8;
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sk += red_k[s * LR + tid];
        sq += red_q[s * LR + tid];
      }
      const float u = bv * (vv - av * sk);
      us[tid] = u;
      const float ov = a.scale * (av * sq + kq_s[par] * u);
      reinterpret_cast<T*>(a.o)[(t * a.Hv + h) * 128 + tid] = from_f<T>(ov);
    }
    __syncthreads();

    // S <- a S + k u^T
    if (!SVF) {
      const float4 u4 = *reinterpret_cast<const float4*>(&us[4 * lo]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = ks[par][16 * hi + r];
        S[r].x = av * S[r].x + kr * u4.x;
        S[r].y = av * S[r].y + kr * u4.y;
        S[r].z = av * S[r].z + kr * u4.z;
        S[r].w = av * S[r].w + kr * u4.w;
      }
    } else {
      const float4 k4 = *reinterpret_cast<const float4*>(&ks[par][4 * lo]);
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float uc = us[16 * hi + c];
        S[c].x = av * S[c].x + k4.x * uc;
        S[c].y = av * S[c].y + k4.y * uc;
        S[c].z = av * S[c].z + k4.z * uc;
        S[c].w = av * S[c].w + k4.w * uc;
      }
    }
  }

  if (a.ht) {
    float* dst = a.ht + ((int64_t)n * a.Hv + h) * KV;
#pragma unroll
    for (int r = 0; r < 16; ++r) *reinterpret_cast<float4*>(dst + piece(r)) = S[r];
  }
}

gdr_status launch_recurrent(const gdr_problem* p, const void* q, const void* k, const void* v,
                            const void* g, const void* beta, const float* h0, void* o,
                            float* ht, hipStream_t st) {
  RecArgs a;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.h0 = h0; a.ht = ht; a.o = o;
  a.cu = p->cu_seqlens_dev;
  a.N = p->N; a.T = p->T; a.Hq = p->Hq; a.Hv = p->Hv;
  a.g_dtype = (int)p->g_dtype;
  a.qk_norm = p->use_qk_l2norm ? 1 : 0;
  a.beta_mode = (p->beta_sigmoid ? 1 : 0) | (p->neg_eigval ? 2 : 0);
  a.scale = p->scale;
  a.gate_A_log = p->use_gate ? p->gate_A_log : nullptr;
  a.gate_dt_bias = p->use_gate ? p->gate_dt_bias : nullptr;
  if ((int64_t)p->N * p->Hv == 0) return GDR_OK;
  const dim3 grid((unsigned)((int64_t)p->N * p->Hv));
  const bool svf = p->state_v_first != 0;
  if (p->in_dtype == GDR_BF16) {
    if (svf) GDR_LAUNCH("recurrent", (recurrent_kernel<__bf16, true>), grid, dim3(256), st, a);
    else GDR_LAUNCH("recurrent", (recurrent_kernel<__bf16, false>), grid, dim3(256), st, a);
  } else {
    if (svf) GDR_LAUNCH("recurrent", (recurrent_kernel<_Float16, true>), grid, dim3(256), st, a);
    else GDR_LAUNCH("recurrent", (recurrent_kernel<_Float16, false>), grid, dim3(256), st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("recurrent launch failed: %s", hipGetErrorString(e));
    return GDR_ERR_HIP;
  }
  return GDR_OK;
}

}  // namespace gdr
