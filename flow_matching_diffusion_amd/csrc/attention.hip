// Masked GQA flash attention with the sigmoid output gate fused in (gfx950).
//
// Krea2Attention (architecture article §四.3): every query head attends over all L tokens of its
// batch row; query head h reads kv head h / G (K/V heads repeated with repeat_interleave
// semantics); scores are scaled by 1/sqrt(head_dim); a text key j < T is excluded when the mask
// marks it padding; image keys are always valid; the output is multiplied elementwise by
// sigmoid(gate) before the output projection.
//
// Two kernels: attn_bf16_kernel (32x32x16 bf16 matrix cores, the production path) and attn_kernel
// (16x16 blocks, used for float32 operands).
//
// attn_kernel: one workgroup = (batch row, kv head, block of query rows). Its 4 waves cover the G query heads
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
#include "k2_tiles.h"

namespace k2 {


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
  K2_LDS_CHECK(sizeof(sK) + sizeof(sV) + sizeof(sBits), 1);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int head = kvh * G + (wave % G);
  const int q0 = blockIdx.x * BQ + (wave / G) * 64;
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const uint4 zero = {0u, 0u, 0u, 0u};

  // Block-causal restriction: query i sees keys j <= reach[i], non-decreasing in i, so the
  // workgroup's first and last queries bound which tiles need it and where the keys end.
  const int qlo = blockIdx.x * BQ;
  int kmin = L - 1, kmax = L - 1;
  int rq[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) rq[qb] = L - 1;
  if (p.reach) {
    kmin = p.reach[qlo];
    kmax = p.reach[min(qlo + BQ, L) - 1];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) rq[qb] = p.reach[min(q0 + qb * 16 + col, L - 1)];
  }

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
  const rsrc_t kr = make_rsrc((const T*)p.k + ((size_t)b * L * ldk + kvh * HD),
                              ((size_t)(L - 1) * ldk + HD) * sizeof(T));
  const T* vbase = (const T*)p.vt + (size_t)(b * p.nkv + kvh) * HD * p.ldvt;
  const rsrc_t vr = make_rsrc(vbase, (size_t)HD * p.ldvt * sizeof(T));
  const int kc = tid % CPRK, krow = tid / CPRK;  // K: rows krow + i * KSTEP
  const int vc = tid % CPRV, vrow = tid / CPRV;  // V^T: rows vrow + i * VSTEP
  constexpr int KSTEP = 256 / CPRK, VSTEP = 256 / CPRV;

  uint4 rk[K_LD], rv[V_LD];
#define K2_ATT_GLOAD(t)                                                                            \
  do {                                                                                             \
    const int t0_ = (t) * KT;                                                                      \
    _Pragma("unroll") for (int i = 0; i < K_LD; ++i)                                               \
      rk[i] = bload(kr, (uint32_t)(((t0_ + krow + i * KSTEP) * ldk + kc * EPC) * sizeof(T))); \
    const int k0_ = t0_ + vc * EPC;                                                                \
    _Pragma("unroll") for (int i = 0; i < V_LD; ++i) {                                             \
      const uint32_t off_ = k0_ < L ? (uint32_t)(((vrow + i * VSTEP) * p.ldvt + k0_) * sizeof(T)) : 0x80000000u; \
      rv[i] = bload(vr, off_);                                                                \
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
  const int nt = (kmax + KT) / KT;  // tiles holding keys 0 .. kmax
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
    if (p.reach && t0 + KT - 1 > kmin) {  // keys past some query's reach
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t0 + 8 * grp + 4 * kb + r;
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            if (key > rq[qb]) s[kb][qb][r] = -INFINITY;
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
    if (p.lse && grp == 0)  // log-sum-exp in base 2 of the scaled scores, for the backward
      p.lse[((size_t)b * p.nh + head) * L + row] = lsum > 0.0f ? m_i[qb] + __log2f(lsum) : INFINITY;
    const size_t base = (size_t)(b * L + row) * ldq + head * HD;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int d0 = hb * 16 + 4 * grp;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gv = to_f(gp[base + d0 + r]);
        // the attention output is a T tensor (bf16 in the bf16 model); the gate multiplies that
        const float ov = to_f(to_t<T>(o[hb][qb][r] * inv));
        if (p.o_pre) ((T*)p.o_pre)[base + d0 + r] = to_t<T>(ov);
        op[base + d0 + r] = to_t<T>(ov * sigmoidf_(gv));
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// attn_bf16_kernel: one workgroup = (batch row, kv head, block of query rows); each of its 4 waves
// owns 32 query rows of one of the G query heads that share the kv head, so every K / V^T tile
// staged in LDS serves all of them. A wave needs under 256 registers, so two workgroups share a
// compute unit and one's softmax overlaps the other's matrix-core work.
//
// Keys come in tiles of 64, streamed by buffer->LDS DMA into two stages. Per tile and 32-key
// block, S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys along rows, the wave's 32 queries along
// columns): a lane holds one query's scores, and the lane 32 apart holds the rest of that query's
// keys, so the row max is an in-lane max plus one exchange. K rows enter the MFMA in a permuted
// order (bits 2 and 3 of the row index swapped) so that accumulator entries 8s'..8s'+7 of lane l are
// keys 16s' + 8(l/32) + 0..7: packed to bf16 they are exactly the B operand (P^T) of
// O^T += V^T P^T for k-step s', and P never leaves registers. V^T (written transposed by the
// projection epilogue) gives contiguous A fragments.
//
// LDS: K rows are 256 bytes (16 chunks) stored at chunk c ^ (row & 15); V^T rows are 128 bytes (8
// chunks) at chunk c ^ swz128(d). Both make the fragment reads (32 rows x 2 chunks) and the DMA
// writes conflict-free.
// Softmax runs in base 2: p = exp2(s * log2(e)/sqrt(hd) - m), one fused multiply-add before exp2.
// The running maximum is rescaled lazily (see above). Text-key validity is kept per 64-key tile.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int swz_k256(int row) { return row & 15; }
__device__ __forceinline__ int swz_v128(int d) { return (d >> 1) & 7; }
// accumulator row -> key of a 32-key block (bits 2 and 3 swapped; an involution)
__device__ __forceinline__ int kperm(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }
// max over lanes l and l ^ 32: v_permlane32_swap of two copies hands every lane both halves'
// values, with no LDS traffic (a shuffle would wait on the fragment reads in flight)
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int kMaxTextTiles64 = 256;  // 64-key text tiles: text tokens up to 16384

template <int HD, int G>
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnArgs p, float scale_log2) {
  constexpr int KT = 64;              // keys per tile
  constexpr int KCH = HD / 8;         // 16-byte chunks per K row
  constexpr int VCH = KT / 8;         // chunks per V^T row
  constexpr int NS = HD / 16;         // k16 steps over head_dim
  constexpr int NHB = HD / 32;        // 32-row head-dim blocks of O^T
  constexpr int WPH = 4 / G;          // waves per query head
  constexpr int BQ = 32 * WPH;        // query rows per workgroup
  constexpr int K_DMA = KT * KCH / 256;  // 1 KB DMA instructions per wave for the K tile
  constexpr int V_DMA = HD * VCH / 256;  // ... and for the V^T tile
  constexpr float kRescale = 8.0f;
  constexpr int RA = 4;               // fragment read-ahead (matrix-core instructions)
  static_assert(KCH == 16 || KCH == 8, "head_dim 128 or 64");

  // two stages each of K and V^T, as separate arrays: the compiler then sees that a DMA into one
  // stage cannot alias reads of the other and does not wait for the DMA before those reads
  __shared__ uint4 sK0[KT * KCH], sK1[KT * KCH];
  __shared__ uint4 sV0[HD * VCH], sV1[HD * VCH];
  __shared__ uint64_t sBits[kMaxTextTiles64];
  K2_LDS_CHECK(sizeof(sK0) + sizeof(sK1) + sizeof(sV0) + sizeof(sV1) + sizeof(sBits), 2);  // 2 per CU
#define K2_SK(st) ((st) ? sK1 : sK0)
#define K2_SV(st) ((st) ? sV1 : sV0)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = p.L, T_ = p.T;
  // (batch row, kv head, query block) items in that order, each XCD taking a contiguous range of
  // every batch row's items (xcd_item_rows), so that the workgroups running together on an XCD share
  // K / V^T in its L2 (dealt round-robin, all eight XCDs streamed the same K / V^T into their own
  // L2s) and every XCD gets the same share of each batch row, whose text padding makes its items
  // cheaper or dearer (one contiguous range of all items gave the first half of the XCDs one batch
  // row and the second half the other)
  const int nqb = (L + BQ - 1) / BQ;
  const int item = xcd_item_rows(blockIdx.x, nqb * p.nkv, p.B);
  const int qb = item % nqb, kvh = (item / nqb) % p.nkv, b = item / nqb / p.nkv;
  const int head = kvh * G + wave % G;
  const int q0 = qb * BQ + (wave / G) * 32;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const int h32 = lane >> 5, c32 = lane & 31;

  // Block-causal restriction: query i sees keys j <= reach[i], non-decreasing in i, so the
  // workgroup's first and last queries bound which tiles need it and where the keys end; rq is
  // this lane's query's reach.
  const int qlo = qb * BQ;
  int kmin = L - 1, kmax = L - 1, rq = L - 1;
  if (p.reach) {
    kmin = p.reach[qlo];
    kmax = p.reach[min(qlo + BQ, L) - 1];
    rq = p.reach[min(q0 + c32, L - 1)];
  }

  // Q^T fragments (B operand of S^T = K Q^T): lane l holds query q0 + l%32, head dims 16s + 8(l/32)..+7;
  // loaded first, so that their latency overlaps the validity bits below
  bf16x8 qf[NS];
  {
    const int row = q0 + c32;
    const bf16* src = (const bf16*)p.q + (size_t)(b * L + (row < L ? row : 0)) * ldq + head * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = row < L ? *(const bf16x8*)(src + 16 * s + 8 * h32) : bf16x8{};
  }

  // validity bits of the text tiles (bit j: key 64t + j is a valid key)
  const int ntt = (T_ + KT - 1) / KT;
  for (int u = wave; u < ntt; u += 4) {
    const int key = u * KT + lane;
    const bool ok = key < L && (key >= T_ || !p.mask || p.mask[(size_t)b * T_ + key] != 0);
    const uint64_t bits = __ballot(ok);
    if (lane == 0) sBits[u] = bits;
  }

  // DMA duties. K: wave w moves tile rows 16w.. (hd 128: 4 blocks of 4 rows; hd 64: 2 blocks of 8).
  // V^T: wave w moves head-dim rows HD/4*w .. (blocks of 8 rows).
  constexpr int KRB = 1024 / (KCH * 16);  // K rows per DMA block
  const rsrc_t kr = make_rsrc((const bf16*)p.k + ((size_t)b * L * ldk + kvh * HD),
                              ((size_t)(L - 1) * ldk + HD) * sizeof(bf16));
  const rsrc_t vr = make_rsrc((const bf16*)p.vt + (size_t)(b * p.nkv + kvh) * HD * p.ldvt,
                              (size_t)HD * p.ldvt * sizeof(bf16));
  uint32_t kvo[K_DMA], vvo[V_DMA];
#pragma unroll
  for (int j = 0; j < K_DMA; ++j) {
    const int row = (wave * K_DMA + j) * KRB + lane / KCH, pc = lane % KCH;
    kvo[j] = (uint32_t)(row * ldk + (pc ^ (swz_k256(row) & (KCH - 1))) * 8) * sizeof(bf16);
  }
#pragma unroll
  for (int j = 0; j < V_DMA; ++j) {
    const int d = (wave * V_DMA + j) * 8 + lane / 8, pc = lane % 8;
    vvo[j] = (uint32_t)(d * p.ldvt + (pc ^ swz_v128(d)) * 8) * sizeof(bf16);
  }
  // DMA of tile t's K rows / V^T columns into stage st (a t past the last tile reads zeros or
  // in-range padding and is never used)
  auto issue_k = [&](int st, int t, int j) {
    dma16(kr, K2_SK(st) + (wave * K_DMA + j) * 64, kvo[j] + (uint32_t)(t * KT * ldk) * sizeof(bf16));
  };
  auto issue_v = [&](int st, int t, int j) {
    dma16(vr, K2_SV(st) + (wave * V_DMA + j) * 64, vvo[j] + (uint32_t)(t * KT) * sizeof(bf16));
  };
  // keys past L in the last tile: V^T columns there hold whatever the workspace held; zero them
  auto zero_tail = [&](int st, int t) {
    const int valid = L - t * KT;  // 0 < valid < KT
    for (int i = tid; i < HD * VCH; i += 256) {
      const int d = i / VCH, pc = i % VCH, k0 = (pc ^ swz_v128(d)) * 8;
      if (k0 + 8 > valid) {
        uint4 v = K2_SV(st)[i];
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + e >= valid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        K2_SV(st)[i] = uint4{w[0], w[1], w[2], w[3]};
      }
    }
  };

  f32x16 o[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[hb][r] = 0.0f;
  float m_i = -INFINITY, l_i = 0.0f;

  // fragment read offsets (uint4 units): K row kperm(l%32) of a 32-key block, V^T row d = l%32
  const int krow = kperm(c32), ksw = swz_k256(krow) & (KCH - 1);
  const int vsw = swz_v128(c32);
#define K2_KFRAG(sk, i) __builtin_bit_cast(bf16x8, (sk)[(32 * ((i) & 1) + krow) * KCH + ((2 * ((i) >> 1) + h32) ^ ksw)])
#define K2_VFRAG(sv, i) __builtin_bit_cast(bf16x8, (sv)[(32 * ((i) % NHB) + c32) * VCH + ((2 * ((i) / NHB) + h32) ^ vsw)])
#define K2_FENCE() __builtin_amdgcn_sched_barrier(0)

  __syncthreads();  // sBits
  const int nt = (kmax + KT) / KT;  // tiles holding keys 0 .. kmax
  auto next_tile = [&](int t) {
    while (t < nt && t < ntt && sBits[t] == 0) ++t;
    return t;
  };
  // Software pipeline over the valid key tiles t_0, t_1, ...: iteration i computes S of t_{i+1}
  // (K in stage (i+1)&1) while running the softmax of t_i, then O^T += V^T P^T for t_i (V in stage
  // i&1) while packing P and summing it; the matrix-core work of each phase is interleaved with
  // the other phase's vector work so that the two overlap. DMA during iteration i: K of t_{i+2}
  // into stage i&1 and V of t_{i+1} into stage (i+1)&1; one barrier per iteration.
  int t = next_tile(0);
  if (t >= nt) {  // no valid key at all: the output is zero
    m_i = 0.0f;
  } else {
    int tn = next_tile(t + 1);
#pragma unroll
    for (int j = 0; j < K_DMA; ++j) issue_k(0, t, j);
#pragma unroll
    for (int j = 0; j < V_DMA; ++j) issue_v(0, t, j);
#pragma unroll
    for (int j = 0; j < K_DMA; ++j) issue_k(1, tn, j);
    K2_WAIT_VM(0);
    __syncthreads();
    if (t * KT + KT > L) {
      zero_tail(0, t);
      __syncthreads();
    }
    f32x16 sa[2], sb[2];  // scores of the tile being finished / the next tile, by 32-key block
    {
      const uint4* sk = sK0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sa[kb][r] = 0.0f;
      bf16x8 ring[RA + 1];
#pragma unroll
      for (int i = 0; i < RA; ++i) ring[i] = K2_KFRAG(sk, i);
      K2_FENCE();
#pragma unroll
      for (int i = 0; i < 2 * NS; ++i) {
        if (i + RA < 2 * NS) ring[(i + RA) % (RA + 1)] = K2_KFRAG(sk, i + RA);
        sa[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % (RA + 1)], qf[i >> 1], sa[i & 1], 0, 0, 0);
        K2_FENCE();
      }
    }
    __syncthreads();  // every wave has read K stage 0

    // One iteration: SC holds tile t's raw scores, SN receives tile tn's; st = i & 1.
#define K2_ATT_ITER(SC, SN, st)                                                                    \
    do {                                                                                           \
      const int tnn = tn < nt ? next_tile(tn + 1) : nt;                                            \
      const uint4* skn = K2_SK((st) ^ 1);                                                          \
      const uint4* svc = K2_SV(st);                                                                \
      /* mask tile t (tiles holding padding or the sequence end only): entry r of block kb is */   \
      /* key 32kb + 16(r/8) + 8(l/32) + r%8, i.e. bytes 4kb + l/32 and 4kb + 2 + l/32 */           \
      const int t0 = t * KT;                                                                       \
      const uint64_t vb = t < ntt ? sBits[t] : (t0 + KT <= L ? ~0ull : ((1ull << (L - t0)) - 1ull)); \
      if (vb != ~0ull) {                                                                           \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                         \
          const uint32_t lb = (uint32_t)((vb >> (8 * (4 * kb + h32))) & 0xFFu) |                   \
                              ((uint32_t)((vb >> (8 * (4 * kb + 2 + h32))) & 0xFFu) << 8);         \
          _Pragma("unroll") for (int r = 0; r < 16; ++r) if (!((lb >> r) & 1u)) SC[kb][r] = -INFINITY; \
        }                                                                                          \
      }                                                                                            \
      if (p.reach && t0 + KT - 1 > kmin) { /* keys past some query's reach */                     \
        _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                           \
          _Pragma("unroll") for (int r = 0; r < 16; ++r)                                           \
            if (t0 + 32 * kb + 16 * (r >> 3) + 8 * h32 + (r & 7) > rq) SC[kb][r] = -INFINITY;       \
      }                                                                                            \
      /* phase A: S of tile tn, interleaved with tile t's max, rescale and exponentials; at raised */ \
      /* wave priority, so that the other workgroup's wave on this SIMD (in phase B) fills the gaps */ \
      __builtin_amdgcn_s_setprio(1);                                                               \
      _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                             \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) SN[kb][r] = 0.0f;                           \
      bf16x8 ring[RA + 1];                                                                         \
      _Pragma("unroll") for (int i = 0; i < RA; ++i) ring[i] = K2_KFRAG(skn, i);                   \
      K2_FENCE();                                                                                  \
      float mx = -INFINITY, base = 0.0f;                                                           \
      _Pragma("unroll") for (int i = 0; i < 2 * NS; ++i) {                                         \
        if (i + RA < 2 * NS) ring[(i + RA) % (RA + 1)] = K2_KFRAG(skn, i + RA);                    \
        SN[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % (RA + 1)], qf[i >> 1], SN[i & 1], 0, 0, 0); \
        if (i < K_DMA) issue_k(st, tnn, i);                                                        \
        else if (i < K_DMA + V_DMA) issue_v((st) ^ 1, tn, i - K_DMA);                              \
        if (i < 4) {                                                                               \
          _Pragma("unroll") for (int e = 0; e < 8; ++e) mx = fmaxf(mx, SC[i >> 1][8 * (i & 1) + e]); \
        } else if (i == 4) {                                                                       \
          mx = max_xor32(mx) * scale_log2;                                                         \
          if (__any(mx > m_i + kRescale)) {                                                        \
            const float mnew = fmaxf(m_i, mx);                                                     \
            const float alpha = m_i == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_i - mnew);      \
            l_i *= alpha;                                                                          \
            _Pragma("unroll") for (int hb = 0; hb < NHB; ++hb) o[hb] *= alpha;                     \
            m_i = mnew;                                                                            \
          }                                                                                        \
          base = m_i == -INFINITY ? 0.0f : m_i;                                                    \
        } else {                                                                                   \
          /* 32 exponentials over the remaining 2 NS - 5 instructions */                            \
          constexpr int NX = 2 * NS - 5;                                                           \
          _Pragma("unroll") for (int x = ((i - 5) * 32) / NX; x < ((i - 4) * 32) / NX; ++x)         \
            SC[x >> 4][x & 15] = __builtin_amdgcn_exp2f(fmaf(SC[x >> 4][x & 15], scale_log2, -base)); \
        }                                                                                          \
        K2_FENCE();                                                                                \
      }                                                                                            \
      /* phase B: O^T += V^T P^T for tile t; step j = (kb, h) covers keys 32kb + 16h .. +15, */    \
      __builtin_amdgcn_s_setprio(0);                                                               \
      /* packed just before its first instruction; the row sum runs alongside */                   \
      bf16x8 vring[RA + 1];                                                                        \
      _Pragma("unroll") for (int i = 0; i < RA; ++i) vring[i] = K2_VFRAG(svc, i);                  \
      K2_FENCE();                                                                                  \
      bf16x8 pf;                                                                                   \
      float ls0 = 0.0f, ls1 = 0.0f;                                                                \
      _Pragma("unroll") for (int i = 0; i < 4 * NHB; ++i) {                                        \
        const int j = i / NHB;                                                                     \
        if (i % NHB == 0) {                                                                        \
          float pv[8];                                                                             \
          _Pragma("unroll") for (int e = 0; e < 8; ++e) pv[e] = SC[j >> 1][8 * (j & 1) + e];        \
          pack8(pf, pv);                                                                           \
        }                                                                                          \
        if (i + RA < 4 * NHB) vring[(i + RA) % (RA + 1)] = K2_VFRAG(svc, i + RA);                  \
        o[i % NHB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vring[i % (RA + 1)], pf, o[i % NHB], 0, 0, 0); \
        /* row sum: 32 values over the 4 NHB instructions */                                       \
        _Pragma("unroll") for (int x = (i * 32) / (4 * NHB); x < ((i + 1) * 32) / (4 * NHB); ++x) { \
          if (x & 1) ls1 += SC[x >> 4][x & 15]; else ls0 += SC[x >> 4][x & 15];                    \
        }                                                                                          \
        K2_FENCE();                                                                                \
      }                                                                                            \
      l_i += ls0 + ls1;                                                                            \
      K2_WAIT_VM(0);                                                                               \
      __syncthreads();                                                                             \
      if (tn < nt && tn * KT + KT > L) {                                                           \
        zero_tail((st) ^ 1, tn);                                                                   \
        __syncthreads();                                                                           \
      }                                                                                            \
      t = tn;                                                                                      \
      tn = tnn;                                                                                    \
    } while (0)
    for (;;) {
      K2_ATT_ITER(sa, sb, 0);
      if (t >= nt) break;
      K2_ATT_ITER(sb, sa, 1);
      if (t >= nt) break;
    }
#undef K2_ATT_ITER
  }
#undef K2_FENCE
#undef K2_KFRAG
#undef K2_VFRAG
#undef K2_SK
#undef K2_SV
  // Epilogue. The wave's 32 rows of gate, output (and saved output) go through buffer resources that
  // end at the sequence end (rows past it read zero and their stores are dropped); all gate loads
  // are issued first, so that their latency overlaps the barrier and the staging below.
  constexpr int LPR = HD / 8, RPI = 64 / LPR, NKR = 32 / RPI;  // lanes per row, rows per instruction
  const int rr = lane / LPR, cc = lane % LPR;
  const int nrow = L - q0 < 0 ? 0 : (L - q0 < 32 ? L - q0 : 32);
  const size_t gbase = (size_t)(b * L + q0) * ldq + head * HD;
  const size_t span = nrow ? ((size_t)(nrow - 1) * ldq + HD) * sizeof(bf16) : 0;
  const rsrc_t rg = make_rsrc((const bf16*)p.g + gbase, span);
  const rsrc_t ro = make_rsrc((bf16*)p.og + gbase, span);
  uint4 gq[NKR];
#pragma unroll
  for (int k = 0; k < NKR; ++k) gq[k] = bload(rg, (uint32_t)((RPI * k + rr) * ldq + 8 * cc) * (uint32_t)sizeof(bf16));
  // normalise into this wave's LDS area (the K/V stages are free now): 32 query rows of HD floats,
  // 16-byte chunk c of row r at chunk c ^ (r % 32); then gate and store row-major, HD/8 lanes per
  // query row with 8 head dims each, so the gate reads and output stores cover whole rows
  const float lsum = l_i + __shfl_xor(l_i, 32);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  if (p.lse && h32 == 0 && q0 + c32 < L)  // log-sum-exp in base 2 of the scaled scores, for the backward
    p.lse[((size_t)b * p.nh + head) * L + q0 + c32] = lsum > 0.0f ? m_i + __log2f(lsum) : INFINITY;
  __syncthreads();  // every wave is done with the K/V stages (all DMAs have landed)
  float4* const st = reinterpret_cast<float4*>(wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1);
  static_assert(32 * HD * sizeof(float) <= sizeof(sK0), "staging area");
  constexpr int CPR = HD / 4;  // 16-byte chunks per staged row
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 8 * hb + 2 * j + h32;
      st[c32 * CPR + (c ^ (c32 & (CPR - 1)))] =
          make_float4(o[hb][4 * j] * inv, o[hb][4 * j + 1] * inv, o[hb][4 * j + 2] * inv, o[hb][4 * j + 3] * inv);
    }
  wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
  for (int k = 0; k < NKR; ++k) {
    const int r = RPI * k + rr;
    const uint32_t off = (uint32_t)(r * ldq + 8 * cc) * (uint32_t)sizeof(bf16);
    const float4 a = st[r * CPR + ((2 * cc) ^ (r & (CPR - 1)))];
    const float4 bq = st[r * CPR + ((2 * cc + 1) ^ (r & (CPR - 1)))];
    const bf16x8 gv = __builtin_bit_cast(bf16x8, gq[k]);
    const float v[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
    if (p.o_pre) {
      bf16x8 ov;
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = (bf16)v[e];
      bstore(make_rsrc((bf16*)p.o_pre + gbase, span), off, __builtin_bit_cast(uint4, ov));
    }
    // the attention output is a bf16 tensor in the bf16 model: the gate multiplies the rounded value
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (bf16)((float)(bf16)v[e] * sigmoidf_((float)gv[e]));
    bstore(ro, off, __builtin_bit_cast(uint4, out));
  }
}

// ---------------------------------------------------------------------------------------------
// Short sequences (L <= 32: the layerwise text-fusion stage runs attention over the 12 hidden
// layers of every token, B = batch x tokens sequences). One wave per (batch row, query head), four
// per workgroup, no LDS: the wave loads its Q^T and permuted K fragments straight from memory,
// computes S^T = K Q^T in HD/16 matrix-core steps, takes the softmax in registers (each lane holds
// one query's scores; lanes l and l + 32 split the keys) and forms O^T = V^T P^T with one step per
// 16 keys. Same masking, GQA head map, scale and gate as the tiled kernel.
// ---------------------------------------------------------------------------------------------
constexpr int kShortL = 32;

template <int HD>
__global__ void __launch_bounds__(256) attn_short_kernel(AttnArgs p, float scale_log2) {
  constexpr int NS = HD / 16;   // k16 steps over head_dim
  constexpr int NHB = HD / 32;  // 32-row head-dim blocks of O^T
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= p.B * p.nh) return;  // no barriers below
  const int b = pair / p.nh, head = pair - b * p.nh;
  const int kvh = head / (p.nh / p.nkv);
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const int h32 = lane >> 5, c32 = lane & 31;

  // Q^T (B operand): lane l holds query l%32, head dims 16s + 8(l/32)..+7. K (A operand): lane l
  // holds key kperm(l%32), so that the probabilities a lane ends up with are the P^T operand.
  const int key_l = kperm(c32);
  const bf16* qsrc = (const bf16*)p.q + (size_t)(b * L + (c32 < L ? c32 : 0)) * ldq + head * HD + 8 * h32;
  const bf16* ksrc = (const bf16*)p.k + (size_t)(b * L + (key_l < L ? key_l : 0)) * ldk + kvh * HD + 8 * h32;
  bf16x8 qf[NS], kf[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    qf[st] = c32 < L ? *(const bf16x8*)(qsrc + 16 * st) : bf16x8{};
    kf[st] = key_l < L ? *(const bf16x8*)(ksrc + 16 * st) : bf16x8{};
  }
  // V^T (A operand of O^T += V^T P^T): lane l holds head dim 32hb + l%32, keys 16c + 8(l/32)..+7;
  // keys at or past L read as zero (the workspace there holds anything)
  const int nch = (L + 15) / 16;
  const bf16* vsrc = (const bf16*)p.vt + ((size_t)(b * p.nkv + kvh) * HD + c32) * p.ldvt + 8 * h32;
  bf16x8 vf[2][NHB];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k0 = 16 * c + 8 * h32;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      uint4 v = uint4{0u, 0u, 0u, 0u};
      if (c < nch && k0 < L) {
        v = *(const uint4*)(vsrc + (size_t)32 * hb * p.ldvt + 16 * c);
        if (k0 + 8 > L) v = keep_first<8>(v, L - k0);
      }
      vf[c][hb] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 sacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
  for (int st = 0; st < NS; ++st) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[st], sacc, 0, 0, 0);

  // softmax over keys (base 2): register r holds key kperm(8(r/4) + 4(l/32) + r%4); with the
  // block-causal restriction the lane's query sees keys up to rq only
  const int rq = p.reach ? p.reach[c32 < L ? c32 : L - 1] : L - 1;
  float sc[16];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = kperm(8 * (r >> 2) + 4 * h32 + (r & 3));
    const bool ok = key <= rq && key < L && (key >= T_ || !p.mask || p.mask[(size_t)b * T_ + key] != 0);
    sc[r] = ok ? sacc[r] * scale_log2 : -INFINITY;
    mx = fmaxf(mx, sc[r]);
  }
  mx = max_xor32(mx);
  if (mx == -INFINITY) mx = 0.0f;  // no valid key: every probability is 0 and the output 0
  float ls = 0.0f;
  float pv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    pv[r] = exp2f(sc[r] - mx);
    ls += pv[r];
  }
  f32x16 o[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[hb][r] = 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c >= nch) break;  // wave-uniform
    bf16x8 pf;
    pack8(pf, pv + 8 * c);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) o[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[c][hb], pf, o[hb], 0, 0, 0);
  }

  // normalise, gate, store: lane holds query l%32 and head dims 32hb + 8j + 4(l/32) + 0..3
  const float lsum = ls + __shfl_xor(ls, 32);
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  if (p.lse && h32 == 0 && c32 < L)  // log-sum-exp in base 2 of the scaled scores, for the backward
    p.lse[((size_t)b * p.nh + head) * L + c32] = lsum > 0.0f ? mx + __log2f(lsum) : INFINITY;
  if (c32 < L) {
    const size_t base = (size_t)(b * L + c32) * ldq + head * HD;
    const bf16* gp = (const bf16*)p.g + base;
    bf16* op = (bf16*)p.og + base;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = 32 * hb + 8 * j + 4 * h32;
        const bf16x4 gv = *(const bf16x4*)(gp + d0);
        bf16x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e)  // the gate multiplies the bf16 attention output
          out[e] = (bf16)((float)(bf16)(o[hb][4 * j + e] * inv) * sigmoidf_((float)gv[e]));
        *(bf16x4*)(op + d0) = out;
        if (p.o_pre) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)(o[hb][4 * j + e] * inv);
          *(bf16x4*)((bf16*)p.o_pre + base + d0) = ov;
        }
      }
  }
}

template <int HD>
static hipError_t launch_attn_short(const AttnArgs& p, hipStream_t s) {
  if (p.L <= 0 || p.B <= 0) return hipSuccess;
  // V^T rows must hold the 32 key slots the fragments read, 16-byte aligned
  if (p.L > kShortL || p.ldvt < kShortL || p.ldvt % 8 != 0) return hipErrorInvalidValue;
  const long pairs = (long)p.B * p.nh;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  hipLaunchKernelGGL((attn_short_kernel<HD>), dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, s, p, scale_log2);
  return hipGetLastError();
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

template <int HD, int G>
static hipError_t launch_attn_bf16(const AttnArgs& p, hipStream_t s) {
  constexpr int BQ = 32 * (4 / G);
  if (p.L <= 0 || p.B <= 0) return hipSuccess;
  if (p.T > kMaxTextTiles64 * 64 || p.ldvt % 64 != 0) return hipErrorInvalidValue;
  const long long items = (long long)((p.L + BQ - 1) / BQ) * p.nkv * p.B;
  if (items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)items);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)HD);
  hipLaunchKernelGGL((attn_bf16_kernel<HD, G>), grid, dim3(256), 0, s, p, scale_log2);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t attn_hd(const AttnArgs& p, hipStream_t s) {
  const int G = p.nh / p.nkv;
  if constexpr (sizeof(T) == 2) {
    if (p.L <= kShortL) return launch_attn_short<HD>(p, s);
    if (G == 4) return launch_attn_bf16<HD, 4>(p, s);
    if (G == 2) return launch_attn_bf16<HD, 2>(p, s);
    if (G == 1) return launch_attn_bf16<HD, 1>(p, s);
  } else {
    if (G == 4) return launch_attn<T, HD, 4>(p, s);
    if (G == 2) return launch_attn<T, HD, 2>(p, s);
    if (G == 1) return launch_attn<T, HD, 1>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t attention(int dt, const AttnArgs& p, hipStream_t s) {
  if (p.hd == 128) return dt == DT_BF16 ? attn_hd<bf16, 128>(p, s) : attn_hd<float, 128>(p, s);
  if (p.hd == 64) return dt == DT_BF16 ? attn_hd<bf16, 64>(p, s) : attn_hd<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace k2
