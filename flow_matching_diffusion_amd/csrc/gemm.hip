// Matrix-core GEMMs of the block with fused epilogues (gfx950).
//
//   C[m, n] = sum_k A[m, k] * W[n, k]
// A is row-major (M, K) activations, W holds nn.Linear weights (N, K); both are K-contiguous so no
// transpose is ever needed. fp32 accumulation in both modes.
//
// Tiling: a workgroup computes a BM x BN tile; each wave a WM x WN sub-tile as 16x16 accumulator
// blocks (see k2_device.h for the fragment convention). The k loop stages BK-wide slabs of A and W
// through LDS, double buffered: the next slab is fetched into registers while the current one feeds
// the matrix cores, then written to the other LDS buffer. LDS rows are 128 bytes with an XOR chunk
// swizzle so fragment reads are free of bank conflicts.
//
// Workgroup order: the hardware deals workgroups round-robin to the 8 XCDs, each with its own L2;
// tile ids are remapped so every XCD owns a contiguous range, rastered in groups of 8 tile rows, so
// tiles running together on one XCD share A and W panels in that XCD's L2.
//
// Epilogues (one pass over the accumulators, no extra kernel):
//   Qkvg   — Krea2Attention projections: per-head RMSNorm (1 + w) and 3-axis RoPE on q and k,
//            v written transposed per (batch, kv head) for the attention kernel, gate as is.
//   Swiglu — silu(x Wgate^T) * (x Wup^T); gate and up rows interleave per wave so one lane holds
//            both factors of an output element.
//   Resid  — h_out = h_in + gate_b * acc (gated residual of the block, float32 stream).
//   Plain  — acc + bias to float and/or activation(acc + bias) to the operand dtype, with a row remap
//            (used for img_in / txt_in / final layer / the time MLP).
#include "k2_device.h"
#include "k2_kernels.h"

namespace k2 {

// ---------------------------------------------------------------------------------------------
// Weight-row maps. The loader moves weight rows in aligned groups of G rows (G divides 64); every
// group lies inside one weight matrix, so group(n) returns that matrix's pointer at virtual row n
// and how many of the group's rows exist there (rows past the end read as zero).
// ---------------------------------------------------------------------------------------------
template <typename T>
struct BSegs {
  const T* p[4];
  int start[5];
  int nseg;
  int ldb;
  __device__ __forceinline__ const T* group(int n, int& nvalid) const {
    int s = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < nseg && n >= start[i]) s = i;
    nvalid = start[s + 1] - n;
    return p[s] + (size_t)(n - start[s]) * ldb;
  }
};

template <typename T, int WN>
struct BSwiglu {
  const T* gate;
  const T* up;
  int I;
  int ldb;
  __device__ __forceinline__ const T* group(int n, int& nvalid) const {
    constexpr int HALF = WN / 2;
    const int per = n / WN, jj = n - per * WN;
    const bool is_up = jj >= HALF;
    const int col = per * HALF + (is_up ? jj - HALF : jj);
    nvalid = I - col;
    return (is_up ? up : gate) + (size_t)(col < I ? col : 0) * ldb;
  }
};

// ---------------------------------------------------------------------------------------------
// Epilogues. acc[i][j][r] holds C[row0 + 16 i + 4 (lane / 16) + r][col0 + 16 j + lane % 16].
// ---------------------------------------------------------------------------------------------
template <typename T>
struct EpiResid {
  const float* hin;
  float* hout;
  const float* gate;
  int gate_stride, L, N;
  template <int MI, int NJ>
  __device__ __forceinline__ void apply(const f32x4 (&acc)[MI][NJ], int row0, int col0, int lane, int M) const {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
        if (m >= M) continue;
        const float* gb = gate ? gate + (size_t)(m / L) * gate_stride : nullptr;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = col0 + j * 16 + (lane & 15);
          if (n >= N) continue;
          const size_t idx = (size_t)m * N + n;
          const float gv = gb ? gb[n] : 1.0f;
          hout[idx] = hin[idx] + gv * acc[i][j][r];
        }
      }
  }
};

template <typename T>
struct EpiPlain {
  const float* bias;
  float* outf;
  int ldf;
  T* outt;
  int ldt, act, N, rpb, orpb, ooff;
  template <int MI, int NJ>
  __device__ __forceinline__ void apply(const f32x4 (&acc)[MI][NJ], int row0, int col0, int lane, int M) const {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
        if (m >= M) continue;
        const size_t orow = (size_t)(m / rpb) * orpb + ooff + (m % rpb);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = col0 + j * 16 + (lane & 15);
          if (n >= N) continue;
          const float v = acc[i][j][r] + (bias ? bias[n] : 0.0f);
          if (outf) outf[orow * ldf + n] = v;
          if (outt) outt[orow * ldt + n] = to_t<T>(act ? gelu_tanhf_(v) : v);
        }
      }
  }
};

template <typename T, int WN>
struct EpiSwiglu {
  T* a;
  int I;
  template <int MI, int NJ>
  __device__ __forceinline__ void apply(const f32x4 (&acc)[MI][NJ], int row0, int col0, int lane, int M) const {
    static_assert(NJ * 16 == WN, "wave width");
    const int cbase = (col0 / WN) * (WN / 2);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int col = cbase + j * 16 + (lane & 15);
          if (col >= I) continue;
          a[(size_t)m * I + col] = to_t<T>(siluf_(acc[i][j][r]) * acc[i][j + NJ / 2][r]);
        }
      }
  }
};

template <typename T, int HD>
struct EpiQkvg {
  T* q;
  T* k;
  T* vt;
  T* g;
  const float* wnq;
  const float* wnk;
  const float* rc;
  const float* rs;
  int nq, nk, L, ldvt;
  float eps;
  template <int MI, int NJ>
  __device__ __forceinline__ void apply(const f32x4 (&acc)[MI][NJ], int row0, int col0, int lane, int M) const {
    constexpr int HB = HD / 16;  // 16-column blocks per head
    static_assert(NJ % HB == 0, "a wave covers whole heads");
    const int ntot = 2 * nq + 2 * nk;
#pragma unroll
    for (int h0 = 0; h0 < NJ; h0 += HB) {
      const int nh0 = col0 + h0 * 16;  // first column of this head (wave-uniform)
      if (nh0 >= ntot) break;
      const int seg = nh0 < nq ? 0 : nh0 < nq + nk ? 1 : nh0 < nq + 2 * nk ? 2 : 3;
      if (seg <= 1) {
        T* dst = seg == 0 ? q : k;
        const int ld = seg == 0 ? nq : nk;
        const int cb = seg == 0 ? nh0 : nh0 - nq;
        const float* wn = seg == 0 ? wnq : wnk;
        float wmul[HB];
#pragma unroll
        for (int jj = 0; jj < HB; ++jj) wmul[jj] = 1.0f + (wn ? wn[jj * 16 + (lane & 15)] : 0.0f);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
            float ss = 0.0f;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj) ss += acc[i][h0 + jj][r] * acc[i][h0 + jj][r];
            ss = group16_sum(ss);
            const float inv = rsqrtf(ss * (1.0f / HD) + eps);
            const int l = (m < M ? m : 0) % L;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj) {
              const int d = jj * 16 + (lane & 15);
              float y = acc[i][h0 + jj][r] * inv * wmul[jj];
              const float partner = __shfl_xor(y, 1);
              if (rc) {
                const float c = rc[(size_t)l * (HD / 2) + (d >> 1)];
                const float s = rs[(size_t)l * (HD / 2) + (d >> 1)];
                y = (d & 1) ? partner * s + y * c : y * c - partner * s;
              }
              if (m < M) dst[(size_t)m * ld + cb + d] = to_t<T>(y);
            }
          }
      } else if (seg == 2) {
        const int kvh = (nh0 - nq - nk) / HD;
        const int nkvh = nk / HD;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
            if (m >= M) continue;
            const int b = m / L, l = m - b * L;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj) {
              const int d = jj * 16 + (lane & 15);
              vt[((size_t)(b * nkvh + kvh) * HD + d) * ldvt + l] = to_t<T>(acc[i][h0 + jj][r]);
            }
          }
      } else {
        const int cb = nh0 - nq - 2 * nk;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = row0 + i * 16 + (lane >> 4) * 4 + r;
            if (m >= M) continue;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj) {
              const int d = jj * 16 + (lane & 15);
              g[(size_t)m * nq + cb + d] = to_t<T>(acc[i][h0 + jj][r]);
            }
          }
      }
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Tile order
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void tile_coords(int bid, int nb, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per = nb >> 3, rem = nb & 7, xcd = bid & 7, loc = bid >> 3;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
  constexpr int GM = 8;
  const int group_size = GM * tiles_n;
  const int group = logical / group_size, first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int r = logical - group * group_size;
  tm = first_m + r % gm;
  tn = r / gm;
}

// ---------------------------------------------------------------------------------------------
// Main loop
// ---------------------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // offset past every resource: the load returns zeros

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, size_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <typename T, int BM, int BN, int WM, int WN, class BMap, class Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const T* __restrict__ A, int lda, int M, int K, int Ntot, BMap bmap, Epi epi) {
  constexpr int NWN = BN / WN, NW = (BM / WM) * NWN, NT = NW * 64;
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = 8;               // chunks per 128-byte LDS row
  constexpr int BK = CPR * EPC;        // bf16: 64, fp32: 32
  constexpr int FC = 8 / EPC;          // chunks per 8-element fragment
  constexpr int KS = BK / 32;          // 32-wide k chunks per slab
  constexpr int RSTEP = NT / CPR;      // rows moved by one load instruction of the workgroup
  constexpr int A_LD = BM / RSTEP, B_LD = BN / RSTEP;
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0 && 64 % RSTEP == 0, "tile/thread mismatch");
  constexpr int MI = WM / 16, NJ = WN / 16;
  typedef typename FragOf<T>::type Frag;

  __shared__ uint4 smem[2][(BM + BN) * CPR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (Ntot + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Thread tid moves chunk column c of rows r + i * RSTEP (i < A_LD / B_LD) of each slab.
  const int c = tid & (CPR - 1), r = tid / CPR;
  const rsrc_t ra_src = make_rsrc(A + (size_t)m0 * lda, (size_t)(M - m0) * lda * sizeof(T));
  rsrc_t rb_src[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int n = n0 + i * RSTEP;
    int nvalid = 0;
    const T* base = n < Ntot ? bmap.group(n, nvalid) : A;
    nvalid = n < Ntot ? (nvalid < 0 ? 0 : (nvalid > RSTEP ? RSTEP : nvalid)) : 0;
    rb_src[i] = make_rsrc(base, (size_t)nvalid * bmap.ldb * sizeof(T));
  }
  uint32_t a_off[A_LD], b_off;
  int a_dst[A_LD], b_dst[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int row = r + i * RSTEP;
    a_off[i] = (uint32_t)(row * lda + c * EPC) * sizeof(T);
    a_dst[i] = row * CPR + (c ^ swz8(row));
  }
  b_off = (uint32_t)(r * bmap.ldb + c * EPC) * sizeof(T);
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int row = r + i * RSTEP;
    b_dst[i] = (BM + row) * CPR + (c ^ swz8(row));
  }

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[A_LD], rb[B_LD];
  const int nk = (K + BK - 1) / BK;

#define K2_GLOAD(kt)                                                                         \
  do {                                                                                       \
    const int k0_ = (kt) * BK;                                                               \
    const bool kin_ = k0_ + c * EPC < K;                                                     \
    const uint32_t kb_ = (uint32_t)k0_ * sizeof(T);                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) ra[i] = bload(ra_src, kin_ ? a_off[i] + kb_ : kOOB); \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) rb[i] = bload(rb_src[i], kin_ ? b_off + kb_ : kOOB); \
  } while (0)

#define K2_SSTORE(buf)                                                        \
  do {                                                                        \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) smem[buf][a_dst[i]] = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) smem[buf][b_dst[i]] = rb[i]; \
  } while (0)

  K2_GLOAD(0);
  K2_SSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) K2_GLOAD(kt + 1);
    const uint4* sA = smem[buf];
    const uint4* sB = smem[buf] + BM * CPR;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag af[MI], bfr[NJ];
      const int cb = ks * 4 * FC + (lane >> 4) * FC;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = wm * WM + i * 16 + (lane & 15);
#pragma unroll
        for (int f = 0; f < FC; ++f) ((uint4*)&af[i])[f] = sA[row * CPR + ((cb + f) ^ swz8(row))];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int row = wn * WN + j * 16 + (lane & 15);
#pragma unroll
        for (int f = 0; f < FC; ++f) ((uint4*)&bfr[j])[f] = sB[row * CPR + ((cb + f) ^ swz8(row))];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mma16(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) K2_SSTORE(buf ^ 1);
    __syncthreads();
  }
#undef K2_GLOAD
#undef K2_SSTORE
  epi.template apply<MI, NJ>(acc, m0 + wm * WM, n0 + wn * WN, lane, M);
}

// ---------------------------------------------------------------------------------------------
// Launch configurations
// ---------------------------------------------------------------------------------------------
template <typename T> struct Cfg;
template <> struct Cfg<bf16> { static constexpr int BM = 256, BN = 256, WM = 64, WN = 128; };
template <> struct Cfg<float> { static constexpr int BM = 64, BN = 128, WM = 32, WN = 128; };

template <typename T, class BMap, class Epi>
static hipError_t launch(const GemmA& a, int Ntot, const BMap& bmap, const Epi& epi, hipStream_t s) {
  typedef Cfg<T> C;
  constexpr int NT = (C::BM / C::WM) * (C::BN / C::WN) * 64;
  if (a.M <= 0 || Ntot <= 0) return hipSuccess;
  const int tiles = ((a.M + C::BM - 1) / C::BM) * ((Ntot + C::BN - 1) / C::BN);
  hipLaunchKernelGGL((gemm_kernel<T, C::BM, C::BN, C::WM, C::WN, BMap, Epi>), dim3(tiles), dim3(NT), 0, s,
                     (const T*)a.A, a.lda, a.M, a.K, Ntot, bmap, epi);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t qkvg_t(const GemmA& a, const QkvgArgs& p, hipStream_t s) {
  BSegs<T> bm;
  bm.p[0] = (const T*)p.wq; bm.p[1] = (const T*)p.wk; bm.p[2] = (const T*)p.wv; bm.p[3] = (const T*)p.wg;
  bm.start[0] = 0; bm.start[1] = p.nq; bm.start[2] = p.nq + p.nk; bm.start[3] = p.nq + 2 * p.nk;
  bm.start[4] = 2 * p.nq + 2 * p.nk;
  bm.nseg = 4;
  bm.ldb = a.K;
  EpiQkvg<T, HD> e;
  e.q = (T*)p.q; e.k = (T*)p.k; e.vt = (T*)p.vt; e.g = (T*)p.g;
  e.wnq = p.wnq; e.wnk = p.wnk; e.rc = p.rope_cos; e.rs = p.rope_sin;
  e.nq = p.nq; e.nk = p.nk; e.L = p.L; e.ldvt = p.ldvt; e.eps = p.eps;
  return launch<T>(a, 2 * p.nq + 2 * p.nk, bm, e, s);
}

template <typename T>
static hipError_t swiglu_t(const GemmA& a, const SwigluArgs& p, hipStream_t s) {
  constexpr int WN = Cfg<T>::WN;
  BSwiglu<T, WN> bm;
  bm.gate = (const T*)p.wgate; bm.up = (const T*)p.wup; bm.I = p.I; bm.ldb = a.K;
  EpiSwiglu<T, WN> e;
  e.a = (T*)p.a; e.I = p.I;
  const int ntot = ((p.I + WN / 2 - 1) / (WN / 2)) * WN;
  return launch<T>(a, ntot, bm, e, s);
}

template <typename T>
static hipError_t resid_t(const GemmA& a, const ResidArgs& p, hipStream_t s) {
  BSegs<T> bm = {};
  bm.p[0] = (const T*)p.w; bm.start[0] = 0; bm.start[1] = p.N; bm.nseg = 1; bm.ldb = a.K;
  EpiResid<T> e;
  e.hin = p.hin; e.hout = p.hout; e.gate = p.gate; e.gate_stride = p.gate_stride; e.L = p.L; e.N = p.N;
  return launch<T>(a, p.N, bm, e, s);
}

template <typename T>
static hipError_t plain_t(const GemmA& a, const PlainArgs& p, hipStream_t s) {
  BSegs<T> bm = {};
  bm.p[0] = (const T*)p.w; bm.start[0] = 0; bm.start[1] = p.N; bm.nseg = 1; bm.ldb = a.K;
  EpiPlain<T> e;
  e.bias = p.bias; e.outf = p.outf; e.ldf = p.ldf; e.outt = (T*)p.outt; e.ldt = p.ldt; e.act = p.act;
  e.N = p.N; e.rpb = p.rows_per_b; e.orpb = p.out_rows_per_b; e.ooff = p.out_row_off;
  return launch<T>(a, p.N, bm, e, s);
}

hipError_t gemm_qkvg(int dt, const GemmA& a, const QkvgArgs& p, hipStream_t s) {
  if (p.hd == 128) return dt == DT_BF16 ? qkvg_t<bf16, 128>(a, p, s) : qkvg_t<float, 128>(a, p, s);
  if (p.hd == 64) return dt == DT_BF16 ? qkvg_t<bf16, 64>(a, p, s) : qkvg_t<float, 64>(a, p, s);
  return hipErrorInvalidValue;
}
hipError_t gemm_swiglu(int dt, const GemmA& a, const SwigluArgs& p, hipStream_t s) {
  return dt == DT_BF16 ? swiglu_t<bf16>(a, p, s) : swiglu_t<float>(a, p, s);
}
hipError_t gemm_resid(int dt, const GemmA& a, const ResidArgs& p, hipStream_t s) {
  return dt == DT_BF16 ? resid_t<bf16>(a, p, s) : resid_t<float>(a, p, s);
}
hipError_t gemm_plain(int dt, const GemmA& a, const PlainArgs& p, hipStream_t s) {
  return dt == DT_BF16 ? plain_t<bf16>(a, p, s) : plain_t<float>(a, p, s);
}

}  // namespace k2
