// Masked GQA flash attention with the sigmoid output gate fused in (gfx950).
//
// Krea2Attention (architecture article §四.3): every query head attends over all L tokens of its
// batch row; query head h reads kv head h / G (K/V heads repeated with repeat_interleave
// semantics); scores are scaled by 1/sqrt(head_dim); a text key j < T is excluded when the mask
// marks it padding; image keys are always valid; the output is multiplied elementwise by
// sigmoid(gate) before the output projection.
//
// One workgroup = (batch row, kv head, block of query rows). Its 4 waves cover the G query heads
// that share the kv head, 64 query rows each, so every K/V tile staged in LDS serves all G heads.
// Per 64-key tile a wave computes S^T = K Q^T (keys along MFMA rows, queries along columns): the
// online-softmax statistics of a query then live in one lane column and need only two cross-group
// shuffles. K rows are fed to the MFMA in a permuted order such that the lane group that ends up
// holding S^T rows 4g..4g+3 of two adjacent 16-key blocks holds 8 consecutive keys; those 8
// probabilities are exactly the B fragment of O^T += V^T P^T, so P never leaves registers. V comes
// in transposed (written that way by the projection epilogue) so V^T fragments are contiguous.
// Tiles whose keys are all padding are skipped.
#include "k2_device.h"
#include "k2_kernels.h"

namespace k2 {

// 16 keys read together by a lane group (key = 32c + 8(r/4) + 4e + r%4) -> distinct chunk slots.
__device__ __forceinline__ int swz_key(int key) { return (key & 3) | ((key >> 1) & 12); }

template <typename T, int HD, int G>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs p, float scale_log2) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int FC = 8 / EPC;          // chunks per 8-element fragment
  constexpr int KT = 64;               // keys per tile
  constexpr int CPRK = HD / EPC;       // chunks per key row of the K tile
  constexpr int CPRV = KT / EPC;       // chunks per head-dim row of the V^T tile
  constexpr int K_CH = KT * CPRK, V_CH = HD * CPRV;
  constexpr int K_LD = K_CH / 256, V_LD = V_CH / 256;
  constexpr int WPH = 4 / G;           // waves per query head
  constexpr int BQ = 64 * WPH;         // query rows per workgroup
  constexpr int NHB = HD / 16;
  constexpr int NKS = HD / 32;
  typedef typename FragOf<T>::type Frag;

  __shared__ uint4 sK[2][K_CH];
  __shared__ uint4 sV[2][V_CH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int head = kvh * G + (wave % G);
  const int q0 = blockIdx.x * BQ + (wave / G) * 64;
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const T* qp = (const T*)p.q;
  const T* kp = (const T*)p.k;
  const T* vp = (const T*)p.vt + (size_t)(b * p.nkv + kvh) * HD * p.ldvt;
  const uint8_t* mrow = p.mask ? p.mask + (size_t)b * T_ : nullptr;
  const uint4 zero = {0u, 0u, 0u, 0u};

  // Q^T fragments stay in registers for the whole key loop.
  Frag qf[4][NKS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int row = q0 + qb * 16 + col;
    const T* src = qp + (size_t)(b * L + (row < L ? row : 0)) * ldq + head * HD;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int f = 0; f < FC; ++f) {
        const int ch = ks * 4 * FC + grp * FC + f;
        ((uint4*)&qf[qb][ks])[f] = row < L ? *(const uint4*)(src + ch * EPC) : zero;
      }
  }

  auto key_ok = [&](int key) -> bool { return key < L && (key >= T_ || !mrow || mrow[key] != 0); };
  const int nt = (L + KT - 1) / KT;
  auto next_needed = [&](int t) -> int {  // wave-uniform; identical in every wave
    for (; t < nt; ++t)
      if (__ballot(key_ok(t * KT + lane))) break;
    return t;
  };

  uint4 rk[K_LD], rv[V_LD];
  auto gload = [&](int t) {
    const int t0 = t * KT;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int qc = tid + i * 256, key = qc / CPRK, c = qc % CPRK, gk = t0 + key;
      rk[i] = gk < L ? *(const uint4*)(kp + (size_t)(b * L + gk) * ldk + kvh * HD + c * EPC) : zero;
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int qc = tid + i * 256, d = qc / CPRV, c = qc % CPRV, k0 = t0 + c * EPC;
      const T* src = vp + (size_t)d * p.ldvt + k0;
      if (k0 + EPC <= L) {
        rv[i] = *(const uint4*)src;
      } else {
        T tmp[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) tmp[e] = (k0 + e < L) ? src[e] : to_t<T>(0.0f);
        rv[i] = *(const uint4*)tmp;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int qc = tid + i * 256, key = qc / CPRK, c = qc % CPRK;
      sK[buf][key * CPRK + (c ^ (swz_key(key) & (CPRK - 1)))] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int qc = tid + i * 256, d = qc / CPRV, c = qc % CPRV;
      sV[buf][d * CPRV + (c ^ (swz8(d) & (CPRV - 1)))] = rv[i];
    }
  };

  f32x4 o[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) o[hb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_i[4], l_i[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    m_i[qb] = -INFINITY;
    l_i[qb] = 0.0f;
  }

  auto compute = [&](int buf, int t) {
    // S^T = K Q^T over this tile
    f32x4 s[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      Frag kf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = 32 * (kb >> 1) + 8 * (col >> 2) + 4 * (kb & 1) + (col & 3);
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          const int ch = ks * 4 * FC + grp * FC + f;
          ((uint4*)&kf[kb])[f] = sK[buf][key * CPRK + (ch ^ (swz_key(key) & (CPRK - 1)))];
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) s[kb][qb] = mma16(s[kb][qb], kf[kb], qf[qb][ks]);
    }

    // key validity of this tile, one bit per key
    const int t0 = t * KT;
    const uint64_t vbits = __ballot(key_ok(t0 + lane));

    // online softmax (base 2), per query column
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + r;
          const float v = ((vbits >> kk) & 1) ? s[kb][qb][r] * scale_log2 : -INFINITY;
          s[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = across_groups_max(mx);
      const float mnew = fmaxf(m_i[qb], mx);
      const float base = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = exp2f(m_i[qb] - base);
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = exp2f(s[kb][qb][r] - base);
          s[kb][qb][r] = pv;
          rs += pv;
        }
      l_i[qb] = l_i[qb] * alpha + rs;
      m_i[qb] = mnew;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) o[hb][qb] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      Frag pf[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        float tmp[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tmp[r] = s[2 * c2][qb][r];
          tmp[4 + r] = s[2 * c2 + 1][qb][r];
        }
        pack8(pf[qb], tmp);
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        Frag vf;
        const int d = hb * 16 + col;
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          const int ch = (c2 * 32 + 8 * grp) / EPC + f;
          ((uint4*)&vf)[f] = sV[buf][d * CPRV + (ch ^ (swz8(d) & (CPRV - 1)))];
        }
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) o[hb][qb] = mma16(o[hb][qb], vf, pf[qb]);
      }
    }
  };

  int t = next_needed(0);
  if (t < nt) {
    gload(t);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (t < nt) {
    const int tn = next_needed(t + 1);
    if (tn < nt) gload(tn);
    compute(buf, t);
    if (tn < nt) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    t = tn;
  }

  // normalise, gate, store: lane holds 4 consecutive head-dim values of one query row
  const T* gp = (const T*)p.g;
  T* op = (T*)p.og;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const float lsum = across_groups_sum(l_i[qb]);
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
    const int row = q0 + qb * 16 + col;
    if (row >= L) continue;
    const size_t base = (size_t)(b * L + row) * ldq + head * HD;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int d0 = hb * 16 + 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = to_f(gp[base + d0 + r]);
        op[base + d0 + r] = to_t<T>(o[hb][qb][r] * inv * sigmoidf_(gv));
      }
    }
  }
}

template <typename T, int HD, int G>
static hipError_t launch_attn(const AttnArgs& p, hipStream_t s) {
  constexpr int BQ = 64 * (4 / G);
  if (p.L <= 0 || p.B <= 0) return hipSuccess;
  dim3 grid((p.L + BQ - 1) / BQ, p.nkv, p.B);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  hipLaunchKernelGGL((attn_kernel<T, HD, G>), grid, dim3(256), 0, s, p, scale_log2);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t attn_hd(const AttnArgs& p, hipStream_t s) {
  const int G = p.nh / p.nkv;
  if (G == 4) return launch_attn<T, HD, 4>(p, s);
  if (G == 2) return launch_attn<T, HD, 2>(p, s);
  if (G == 1) return launch_attn<T, HD, 1>(p, s);
  return hipErrorInvalidValue;
}

hipError_t attention(int dt, const AttnArgs& p, hipStream_t s) {
  if (p.hd == 128) return dt == DT_BF16 ? attn_hd<bf16, 128>(p, s) : attn_hd<float, 128>(p, s);
  if (p.hd == 64) return dt == DT_BF16 ? attn_hd<bf16, 64>(p, s) : attn_hd<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace k2
