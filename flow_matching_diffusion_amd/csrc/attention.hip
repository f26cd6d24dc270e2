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
// Per key tile a wave computes S^T = K Q^T (keys along MFMA rows, queries along columns): the
// online-softmax statistics of a query then live in one lane column and need only two cross-group
// shuffles. K rows are fed to the MFMA in a permuted order such that the lane group that ends up
// holding S^T rows 4g..4g+3 of the tile's two 16-key blocks holds 8 consecutive keys; those 8
// probabilities are exactly the B fragment of O^T += V^T P^T, so P never leaves registers. V comes
// in transposed (written that way by the projection epilogue) so V^T fragments are contiguous.
//
// Keys come in tiles of 32. Key validity of the text tiles is computed once per workgroup into
// LDS; tiles whose keys are all padding are skipped, and only tiles holding padding or the sequence
// end pay for masking.
// The running maximum is rescaled lazily: O and the row sums are only rescaled when some query's
// maximum grew by more than 2^8 since the last rescale (exp2 of scores up to 2^8 stays exact in
// the float32 sum and the bf16 P operand), which the final division by the row sum undoes exactly.
#include "k2_device.h"
#include "k2_kernels.h"

namespace k2 {

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t attn_rsrc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 attn_bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 16 keys read together by a lane group (key = 32c + 8(r/4) + 4e + r%4) -> distinct chunk slots.
__device__ __forceinline__ int swz_key(int key) { return (key & 3) | ((key >> 1) & 12); }

constexpr int kMaxTextTiles = 512;  // 32-key text tiles: text tokens up to 16384

// Keep the first n (0 < n < EPC) elements of a 16-byte chunk of EPC elements, zero the rest.
template <int EPC>
__device__ __forceinline__ uint4 keep_first(uint4 v, int n) {
  constexpr int BITS = 128 / EPC;  // bits per element: 16 (bf16) or 32 (fp32)
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 32 / BITS; ++e)
      if (i * (32 / BITS) + e < n) m |= (BITS == 32 ? 0xFFFFFFFFu : (0xFFFFu << (e * BITS)));
    w[i] &= m;
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// V^T tile rows hold the 32 keys of a tile: 64 bytes (bf16, 4 chunks) or 128 bytes (fp32, 8 chunks).
// 16 consecutive rows read at one chunk land in distinct bank slots (128- or 256-byte LDS cycles).
template <int CPR>
__device__ __forceinline__ int swz_v(int d) {
  return CPR == 4 ? (((d >> 2) ^ (d >> 1)) & 3) : (swz8(d) & (CPR - 1));
}

template <typename T, int HD, int G>
__global__ void __launch_bounds__(256) attn_kernel(AttnArgs p, float scale_log2) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int FC = 8 / EPC;          // chunks per 8-element fragment
  constexpr int KT = 32;               // keys per tile
  constexpr int CPRK = HD / EPC;       // chunks per key row of the K tile
  constexpr int CPRV = KT / EPC;       // chunks per head-dim row of the V^T tile
  constexpr int K_CH = KT * CPRK, V_CH = HD * CPRV;
  constexpr int K_LD = K_CH / 256, V_LD = V_CH / 256;
  static_assert(K_CH % 256 == 0 && V_CH % 256 == 0, "tile/thread mismatch");
  constexpr int WPH = 4 / G;           // waves per query head
  constexpr int BQ = 64 * WPH;         // query rows per workgroup
  constexpr int NHB = HD / 16;
  constexpr int NKS = HD / 32;
  constexpr float kRescale = 8.0f;     // log2 growth of the maximum that forces a rescale
  typedef typename FragOf<T>::type Frag;

  __shared__ uint4 sK[2][K_CH];
  __shared__ uint4 sV[2][V_CH];
  __shared__ uint32_t sBits[kMaxTextTiles];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int head = kvh * G + (wave % G);
  const int q0 = blockIdx.x * BQ + (wave / G) * 64;
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const uint4 zero = {0u, 0u, 0u, 0u};

  // Validity bits of the 32-key tiles that hold text keys (bit j: key t*32 + j is a valid key);
  // one wave ballot covers two tiles.
  const int ntt = (T_ + KT - 1) / KT;
  for (int u = wave; 2 * u < ntt; u += 4) {
    const int key = u * 64 + lane;
    const bool ok = key < L && (key >= T_ || !p.mask || p.mask[(size_t)b * T_ + key] != 0);
    const uint64_t bits = __ballot(ok);
    if (lane == 0) {
      sBits[2 * u] = (uint32_t)bits;
      if (2 * u + 1 < ntt) sBits[2 * u + 1] = (uint32_t)(bits >> 32);
    }
  }

  // Q^T fragments stay in registers for the whole key loop.
  const T* qp = (const T*)p.q;
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

  // K rows of this (batch, kv head); V^T rows (head dims) of length ldvt.
  const rsrc_t kr = attn_rsrc((const T*)p.k + ((size_t)b * L * ldk + kvh * HD),
                              ((size_t)(L - 1) * ldk + HD) * sizeof(T));
  const T* vbase = (const T*)p.vt + (size_t)(b * p.nkv + kvh) * HD * p.ldvt;
  const rsrc_t vr = attn_rsrc(vbase, (size_t)HD * p.ldvt * sizeof(T));
  const int kc = tid % CPRK, krow = tid / CPRK;  // K: rows krow + i * KSTEP
  const int vc = tid % CPRV, vrow = tid / CPRV;  // V^T: rows vrow + i * VSTEP
  constexpr int KSTEP = 256 / CPRK, VSTEP = 256 / CPRV;

  uint4 rk[K_LD], rv[V_LD];
#define K2_ATT_GLOAD(t)                                                                            \
  do {                                                                                             \
    const int t0_ = (t) * KT;                                                                      \
    _Pragma("unroll") for (int i = 0; i < K_LD; ++i)                                               \
      rk[i] = attn_bload(kr, (uint32_t)(((t0_ + krow + i * KSTEP) * ldk + kc * EPC) * sizeof(T))); \
    const int k0_ = t0_ + vc * EPC;                                                                \
    _Pragma("unroll") for (int i = 0; i < V_LD; ++i) {                                             \
      const uint32_t off_ = k0_ < L ? (uint32_t)(((vrow + i * VSTEP) * p.ldvt + k0_) * sizeof(T)) : 0x80000000u; \
      rv[i] = attn_bload(vr, off_);                                                                \
      if (k0_ + EPC > L && k0_ < L) rv[i] = keep_first<EPC>(rv[i], L - k0_);                        \
    }                                                                                              \
  } while (0)
#define K2_ATT_SSTORE(buf)                                                                         \
  do {                                                                                             \
    _Pragma("unroll") for (int i = 0; i < K_LD; ++i) {                                             \
      const int key_ = krow + i * KSTEP;                                                           \
      sK[buf][key_ * CPRK + (kc ^ (swz_key(key_) & (CPRK - 1)))] = rk[i];                          \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < V_LD; ++i) {                                             \
      const int d_ = vrow + i * VSTEP;                                                             \
      sV[buf][d_ * CPRV + (vc ^ swz_v<CPRV>(d_))] = rv[i];                                         \
    }                                                                                              \
  } while (0)

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

  __syncthreads();  // sBits ready
  const int nt = (L + KT - 1) / KT;
  int t = 0;
  while (t < nt && t < ntt && sBits[t] == 0) ++t;
  if (t < nt) {
    K2_ATT_GLOAD(t);
    K2_ATT_SSTORE(0);
  }
  __syncthreads();
  int buf = 0;
  while (t < nt) {
    int tn = t + 1;
    while (tn < nt && tn < ntt && sBits[tn] == 0) ++tn;  // skip tiles of padding only
    if (tn < nt) K2_ATT_GLOAD(tn);
    const int t0 = t * KT;

    // S^T = K Q^T over this tile: block kb, lane row 4g + r holds key 8g + 4kb + r
    f32x4 s[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      Frag kf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = 8 * (col >> 2) + 4 * kb + (col & 3);
#pragma unroll
        for (int f = 0; f < FC; ++f) {
          const int ch = ks * 4 * FC + grp * FC + f;
          ((uint4*)&kf[kb])[f] = sK[buf][key * CPRK + (ch ^ (swz_key(key) & (CPRK - 1)))];
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) s[kb][qb] = mma16(s[kb][qb], kf[kb], qf[qb][ks]);
    }

    // scale to base 2; mask only tiles with padding or the sequence end
    const uint32_t vbits = t < ntt ? sBits[t] : (t0 + KT <= L ? ~0u : ((1u << (L - t0)) - 1u));
    if (vbits == ~0u) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) s[kb][qb] *= scale_log2;
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (vbits >> (8 * grp + 4 * kb + r)) & 1u;
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) s[kb][qb][r] = ok ? s[kb][qb][r] * scale_log2 : -INFINITY;
        }
    }

    // online softmax with lazy rescaling
    float mt[4];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mt[qb] = across_groups_max(mx);
      grow |= mt[qb] > m_i[qb] + kRescale;
    }
    if (__any(grow)) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const float mnew = fmaxf(m_i[qb], mt[qb]);
        const float alpha = m_i[qb] == -INFINITY ? 0.0f : exp2f(m_i[qb] - mnew);
        l_i[qb] *= alpha;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) o[hb][qb] *= alpha;
        m_i[qb] = mnew;
      }
    }
    Frag pf[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      const float base = m_i[qb] == -INFINITY ? 0.0f : m_i[qb];
      float pv[8];
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pv[4 * kb + r] = exp2f(s[kb][qb][r] - base);
          rs += pv[4 * kb + r];
        }
      l_i[qb] += rs;
      pack8(pf[qb], pv);
    }

    // O^T += V^T P^T: A = V^T rows (head dims), k slots = the lane group's 8 consecutive keys
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      Frag vf;
      const int d = hb * 16 + col;
#pragma unroll
      for (int f = 0; f < FC; ++f) {
        const int ch = grp * FC + f;
        ((uint4*)&vf)[f] = sV[buf][d * CPRV + (ch ^ swz_v<CPRV>(d))];
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) o[hb][qb] = mma16(o[hb][qb], vf, pf[qb]);
    }

    if (tn < nt) K2_ATT_SSTORE(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    t = tn;
  }
#undef K2_ATT_GLOAD
#undef K2_ATT_SSTORE

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
  if (p.T > kMaxTextTiles * 32) return hipErrorInvalidValue;
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
