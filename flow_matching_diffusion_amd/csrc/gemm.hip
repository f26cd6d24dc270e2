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
#include "k2_tiles.h"

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
// Accumulator layouts. Both main loops feed the matrix cores with the weight fragment as the first
// operand and the activation fragment as the second, so the instruction computes a block of C^T and
// each lane ends up holding ONE output row and runs of 4 consecutive output columns:
//   16x16 (fp32 path, v_mfma_f32_16x16x4f32):   lane holds row lane%16, columns 4*(lane/16) + e
//   32x32 (bf16 path, v_mfma_f32_32x32x16_bf16): lane holds row lane%32, columns 8*q + 4*(lane/32) + e
// with e < 4 and q < NQ. A wave's tile is MI x NJ blocks of BS x BS, and
//   acc[i][j][4*q + e] = C[row0 + row(i, lane)][col0 + col(j, q, lane) + e].
// rowsum() adds over the lanes holding the same row.
// ---------------------------------------------------------------------------------------------
template <int BS> struct Lay;
template <> struct Lay<16> {
  typedef f32x4 F;
  static constexpr int NQ = 1;
  __device__ static __forceinline__ int row(int i, int lane) { return 16 * i + (lane & 15); }
  __device__ static __forceinline__ int col(int j, int q, int lane) { return 16 * j + 4 * (lane >> 4); }
  __device__ static __forceinline__ float rowsum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
  }
};
template <> struct Lay<32> {
  typedef f32x16 F;
  static constexpr int NQ = 4;
  __device__ static __forceinline__ int row(int i, int lane) { return 32 * i + (lane & 31); }
  __device__ static __forceinline__ int col(int j, int q, int lane) { return 32 * j + 8 * q + 4 * (lane >> 5); }
  __device__ static __forceinline__ float rowsum(float v) { return v + __shfl_xor(v, 32); }
};

template <class F>
__device__ __forceinline__ float4 quad(const F& a, int q) {
  return make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void st4(bf16* p, float4 v) {
  bf16x4 t;
  t[0] = (bf16)v.x; t[1] = (bf16)v.y; t[2] = (bf16)v.z; t[3] = (bf16)v.w;
  *reinterpret_cast<bf16x4*>(p) = t;
}
// two floats rounded to bf16 (nearest even) and packed, the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
}
__device__ __forceinline__ float4 fma4(float4 g, float4 a, float4 h) {
  return make_float4(h.x + g.x * a.x, h.y + g.y * a.y, h.z + g.z * a.z, h.w + g.w * a.w);
}

// ---------------------------------------------------------------------------------------------
// Epilogues: every access moves 4 consecutive columns (N, I, ld* and all column offsets are
// multiples of 4; the entry points require 16-byte aligned activation, bias and output pointers).
// ---------------------------------------------------------------------------------------------
// Epilogues that read nothing beyond their own arguments stage nothing in LDS.
struct EpiNoStage {
  static constexpr bool kOutStage = false;  // the epilogue takes a per-wave output staging area too
  static constexpr int kOutFloats = 0;
  static constexpr bool kStaged = false;
  static constexpr bool kLdsOut = false;  // the epilogue writes its output through a per-wave LDS area
  static constexpr int kLdsOutFloats = 0;
  static constexpr int stage_floats() { return 0; }
  static constexpr bool kColumnHalves = true;  // a wave 64 columns wide is fine (256x128 half tiles)
  __device__ __forceinline__ bool wants_stage(int) const { return false; }
  __device__ __forceinline__ void stage(float*, int, int, int) const {}
};

// hout = hin + gate[batch] * acc (gated residual; gate NULL means 1). hin may alias hout.
//
// bf16 operands: each 32-row block of the wave's accumulators goes through the wave's LDS area and
// is read back row-major, 32 lanes per 128-column row, so every residual load and store moves whole
// 512-byte row segments (straight from the accumulator layout an instruction touched 32 rows 24 KiB
// apart with 32 bytes each). The next block's residual rows are loaded while the current one is
// written. Everything goes through buffer resources over the wave's rows (rows past M read zero and
// their stores are dropped; columns past N take an offset past every resource) and nothing sits in
// a branch: with the gate loaded per row in a branch, the compiler waited for every memory
// operation in flight (the next block's loads and all earlier stores) before each row's store.
// kWideL (L >= 128, chosen by the host): a wave's 128 rows span at most two batch rows, whose two
// gate vectors are loaded once; otherwise every row's gate is loaded with its residual.
template <typename T, bool kWideL = true>
struct EpiResid : EpiNoStage {
  static constexpr bool kLdsOut = sizeof(T) == 2;
  static constexpr int kPitchF = 132;  // floats per staged row: 128 + 4 of padding
  static constexpr int kLdsOutFloats = sizeof(T) == 2 ? 32 * kPitchF : 0;
  const float* hin;
  float* hout;
  const float* gate;
  int gate_stride, L, N;
  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                        int M, float* stg = nullptr) const {
    constexpr int NQ = LY::NQ, ROWS = MI * (NQ == 1 ? 16 : 32);  // rows of the wave's block
    const int nrow = M - row0 < 0 ? 0 : (M - row0 < ROWS ? M - row0 : ROWS);
    const size_t base = (size_t)row0 * N;
    const rsrc_t rin = make_rsrc(hin + base, (size_t)nrow * N * sizeof(float));
    const rsrc_t rout = make_rsrc(hout + base, (size_t)nrow * N * sizeof(float));
    const int nb = M > 0 ? (M - 1) / L + 1 : 0;  // batch rows the gate holds
    const rsrc_t rg = make_rsrc(gate ? gate : hin, gate && nb ? ((size_t)(nb - 1) * gate_stride + N) * sizeof(float) : 0);
    if constexpr (kLdsOut) {
      static_assert(NQ == 4 && NJ * 32 <= 128 && MI * 32 <= 128, "staged layout: 32x32 blocks, up to 128 x 128 per wave");
      const int hi = lane >> 5, r = lane & 31;   // writer: row r, columns 32 j + 8 q + 4 hi
      const int rr = lane >> 5, ch = lane & 31;  // reader: rows 2 k + rr, columns 4 ch .. 4 ch + 3
      const int n = col0 + 4 * ch;
      const bool colok = ch < 8 * NJ && n < N;  // N is a multiple of 4
      const float4 one = make_float4(1.f, 1.f, 1.f, 1.f);
      // kWideL: gate rows of the first and the last batch row of the wave's rows; rows from
      // `split` on (within the wave's block) take the second
      const int b0 = nrow ? row0 / L : 0, bl = nrow ? (row0 + nrow - 1) / L : 0;
      const int split = (b0 + 1) * L - row0;
      float4 g0 = one, g1 = one;
      if constexpr (kWideL) {
        const float4 g0l = __builtin_bit_cast(float4, bload(rg, colok ? (uint32_t)(b0 * gate_stride + n) * 4u : kOOB));
        const float4 g1l = __builtin_bit_cast(float4, bload(rg, colok ? (uint32_t)(bl * gate_stride + n) * 4u : kOOB));
        g0 = gate ? g0l : one;
        g1 = gate ? g1l : one;
      }
      // residual rows of block i (16 row pairs) and, for !kWideL, their gates; loaded one block ahead
      // for kWideL (at the start of the block otherwise, which keeps that variant's registers)
      float4 hv[2][16], gq[2][16];
      auto load = [&](int s, int i) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int row = 32 * i + 2 * k + rr;
          hv[s][k] = __builtin_bit_cast(float4, bload(rin, colok ? (uint32_t)(row * N + n) * 4u : kOOB));
          if constexpr (!kWideL) {
            const int m = row0 + row < M ? row0 + row : (M > 0 ? M - 1 : 0);
            gq[s][k] = __builtin_bit_cast(float4, bload(rg, colok ? (uint32_t)((m / L) * gate_stride + n) * 4u : kOOB));
          }
        }
      };
      load(0, 0);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if constexpr (kWideL) {
          if (i + 1 < MI) load((i + 1) & 1, i + 1);
        } else if (i > 0) {
          load(i & 1, i);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(stg + r * kPitchF + 32 * j + 8 * q + 4 * hi) = quad(acc[i][j], q);
        wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int sr = 2 * k + rr, row = 32 * i + sr;  // staged row, row of the wave's block
          const float4 v = *reinterpret_cast<const float4*>(stg + sr * kPitchF + 4 * ch);
          float4 gv;
          if constexpr (kWideL) gv = row >= split ? g1 : g0;
          else gv = gate ? gq[i & 1][k] : one;
          bstore(rout, colok ? (uint32_t)(row * N + n) * 4u : kOOB, fma4(gv, v, hv[i & 1][k]));
        }
        wave_lds_sync();  // the next block's writes come after every lane's reads
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = LY::row(i, lane);
        const int m = row0 + r;
        const uint32_t grow = (uint32_t)((m < M ? m : 0) / L) * (uint32_t)gate_stride;
        uint32_t off[NJ][NQ];
        float4 hv[NJ][NQ], gv[NJ][NQ];
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int n = col0 + LY::col(j, q, lane);
            off[j][q] = n < N ? (uint32_t)(r * N + n) * (uint32_t)sizeof(float) : kOOB;
            hv[j][q] = __builtin_bit_cast(float4, bload(rin, off[j][q]));
            gv[j][q] = gate ? __builtin_bit_cast(float4, bload(rg, n < N ? (grow + (uint32_t)n) * 4u : kOOB))
                            : make_float4(1.f, 1.f, 1.f, 1.f);
          }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < NQ; ++q)
            bstore(rout, off[j][q], fma4(gv[j][q], quad(acc[i][j], q), hv[j][q]));
      }
    }
  }
};

// acc + bias into a float output and/or act(acc + bias) into an operand-dtype output, with input
// row m written to output row (m / rpb) * orpb + ooff + m % rpb.
template <typename T>
struct EpiPlain : EpiNoStage {
  const float* bias;
  float* outf;
  int ldf;
  T* outt;
  int ldt, act, N, rpb, orpb, ooff;
  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                        int M, float* stg = nullptr) const {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = row0 + LY::row(i, lane);
      if (m >= M) continue;
      const size_t orow = (size_t)(m / rpb) * orpb + ooff + (m % rpb);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < LY::NQ; ++q) {
          const int n = col0 + LY::col(j, q, lane);
          if (n >= N) continue;
          float4 v = quad(acc[i][j], q);
          if (bias) {
            const float4 b4 = ld4(bias + n);
            v.x += b4.x; v.y += b4.y; v.z += b4.z; v.w += b4.w;
          }
          if (outf) st4(outf + orow * ldf + n, v);
          if (outt) {
            if (act) v = make_float4(gelu_tanhf_(v.x), gelu_tanhf_(v.y), gelu_tanhf_(v.z), gelu_tanhf_(v.w));
            st4(outt + orow * ldt + n, v);
          }
        }
    }
  }
};

// acc into a float32 output only (row m to row m, no bias): the backward's products. bf16: each
// 32-row block of the wave's output (32 rows x WN floats, rows padded to kPitchF) goes through the
// wave's LDS area in the accumulator layout and is read back row-major, 32 lanes per 512-byte row
// segment, so that every store writes whole lines. Stored from the accumulator layout, each
// 16-byte store hit a different row, and the weight-gradient products wrote up to twice their bytes.
template <typename T>
struct EpiPlainF32 : EpiNoStage {
  static constexpr bool kLdsOut = sizeof(T) == 2;
  static constexpr int kPitchF = 132;  // floats per staged row: 128 + 4 of padding
  static constexpr int kLdsOutFloats = sizeof(T) == 2 ? 32 * kPitchF : 0;
  float* outf;
  int ldf, N;
  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                        int M, float* stg = nullptr) const {
    if constexpr (kLdsOut) {
      static_assert(LY::NQ == 4 && NJ * 32 <= 128, "staged layout: 32x32 blocks, up to 128 columns per wave");
      const int hi = lane >> 5, r = lane & 31;  // writer: row r, columns 32 j + 8 q + 4 hi
      const int rr = lane >> 5, ch = lane & 31;  // reader: row 2 k + rr, columns 4 ch .. 4 ch + 3
      const int n = col0 + 4 * ch;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) *reinterpret_cast<float4*>(stg + r * kPitchF + 32 * j + 8 * q + 4 * hi) = quad(acc[i][j], q);
        wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int row = 2 * k + rr;
          const float4 v = *reinterpret_cast<const float4*>(stg + row * kPitchF + 4 * ch);
          const int m = row0 + 32 * i + row;
          if (ch < 8 * NJ && m < M && n < N) st4(outf + (size_t)m * ldf + n, v);  // N is a multiple of 4
        }
        wave_lds_sync();  // the next block's writes come after every lane's reads
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = row0 + LY::row(i, lane);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < LY::NQ; ++q) {
            const int n = col0 + LY::col(j, q, lane);
            if (n < N) st4(outf + (size_t)m * ldf + n, quad(acc[i][j], q));
          }
      }
    }
  }
};

// a = silu(gate) * up; the wave's first WN/2 columns are gate, the last WN/2 the matching up columns.
// kSave: also store float32 copies of the gate and up projections (the backward's recompute); a
// compile-time switch, so that the forward's instantiation carries none of that code.
template <typename T, int WN, bool kSave = false>
struct EpiSwiglu : EpiNoStage {
  // bf16: each 32-row block of the wave's output (32 rows x WN/2 columns) is written to the wave's
  // LDS area in the accumulator layout, then read back row-major, 8 lanes per 128-byte row, so
  // every global store writes whole 128-byte lines. Stored straight from the accumulator layout,
  // an instruction wrote 16 bytes into each of 32 rows 32 KiB apart, and the kernel wrote 2.6x its
  // output to memory (partial lines).
  static constexpr bool kLdsOut = sizeof(T) == 2;
  static constexpr bool kColumnHalves = false;  // gate and up columns pair across the wave's WN
  static constexpr int kPitch = 144;  // bytes per staged row: 128 + 16 of padding
  static constexpr int kLdsOutFloats = sizeof(T) == 2 ? 128 * kPitch / 4 : 0;  // 128 rows per wave
  T* a;
  int I;
  float* gsave;  // kSave only
  float* usave;
  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                        int M, float* stg = nullptr) const {
    static_assert(NJ * (LY::NQ == 1 ? 16 : 32) == WN, "wave width");
    const int cbase = (col0 / WN) * (WN / 2);
    if constexpr (kSave && kLdsOut) {
      // float32 saves through the same LDS area: per 32-row block, gate then up (32 rows x WN/2
      // floats each, rows padded to kSavePitch bytes), read back 16 lanes per 256-byte row so that
      // every store writes whole lines. Stored from the accumulator layout, each 16-byte store hit a
      // different row. The bf16 staging below reuses the area after a wave-scope sync.
      constexpr int kSavePitch = 272;
      static_assert(2 * 32 * kSavePitch <= 4 * kLdsOutFloats, "save staging");
      char* const sm = reinterpret_cast<char*>(stg);
      const int hi = lane >> 5, r = lane & 31;   // writer: row r, columns 8 q + 4 hi of each block
      const int rr = lane >> 4, ch = lane & 15;  // reader: row 4 k + rr, columns 4 ch .. 4 ch + 3
      const int c = cbase + 4 * ch;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // gate, up
          char* const blk = sm + h * 32 * kSavePitch;
#pragma unroll
          for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(blk + r * kSavePitch + 128 * j + 32 * q + 16 * hi) =
                  quad(acc[i][j + h * (NJ / 2)], q);
        }
        wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* const blk = sm + h * 32 * kSavePitch;
          float* const dst = h ? usave : gsave;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int row = 4 * k + rr;
            const float4 v = *reinterpret_cast<const float4*>(blk + row * kSavePitch + 16 * ch);
            const int m = row0 + 32 * i + row;
            if (m < M && c < I) st4(dst + (size_t)m * I + c, v);  // I is a multiple of 4
          }
        }
        wave_lds_sync();  // later writes to the area come after every lane's reads
      }
    } else if constexpr (kSave) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = row0 + LY::row(i, lane);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q = 0; q < LY::NQ; ++q) {
            const int c = cbase + LY::col(j, q, lane);
            if (c >= I) continue;
            st4(gsave + (size_t)m * I + c, quad(acc[i][j], q));
            st4(usave + (size_t)m * I + c, quad(acc[i][j + NJ / 2], q));
          }
      }
    }
    if constexpr (kLdsOut) {
      static_assert(LY::NQ == 4 && WN == 128 && MI * 32 <= 128, "staged layout: 32x32 blocks, 64 bf16 per row");
      char* const sm = reinterpret_cast<char*>(stg);
      const int hi = lane >> 5, r = lane & 31;  // writer: row r, columns 8 q + 4 hi of each block
      const int rr = lane >> 3, ch = lane & 7;  // reader: row 8 k + rr, columns 8 ch .. 8 ch + 7
      const int c = cbase + 8 * ch;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        char* const blk = sm + i * 32 * kPitch;  // blocks do not share LDS: no wait between them
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 g = quad(acc[i][j], q), u = quad(acc[i][j + NJ / 2], q);
            *reinterpret_cast<uint2*>(blk + r * kPitch + 64 * j + 16 * q + 8 * hi) =
                make_uint2(pack_bf16x2(siluf_(g.x) * u.x, siluf_(g.y) * u.y),
                           pack_bf16x2(siluf_(g.z) * u.z, siluf_(g.w) * u.w));
          }
        wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = 8 * k + rr;
          const uint4 v = *reinterpret_cast<const uint4*>(blk + row * kPitch + 16 * ch);
          const int m = row0 + 32 * i + row;
          if (m < M && c < I) {
            T* p = a + (size_t)m * I + c;
            if (c + 8 <= I)
              *reinterpret_cast<uint4*>(p) = v;
            else  // I is a multiple of 4: the last chunk holds 4 columns
              *reinterpret_cast<uint2*>(p) = make_uint2(v.x, v.y);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = row0 + LY::row(i, lane);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
          for (int q = 0; q < LY::NQ; ++q) {
            const int c = cbase + LY::col(j, q, lane);
            if (c >= I) continue;
            const float4 g = quad(acc[i][j], q), u = quad(acc[i][j + NJ / 2], q);
            st4(a + (size_t)m * I + c, make_float4(siluf_(g.x) * u.x, siluf_(g.y) * u.y, siluf_(g.z) * u.z,
                                                   siluf_(g.w) * u.w));
          }
      }
    }
  }
};

// Fused QKV + output-gate projection: per head of q and k, RMSNorm over the head's HD columns
// (weight 1 + w) then rotary embedding on interleaved pairs (2c, 2c+1); v goes out transposed
// (vt[b][kv head][d][token], leading dimension ldvt); the gate projection goes out as is.
// kSave: the backward's recompute also stores raw q / k before their norms (float32), v row-major
// and k after norm and RoPE transposed like vt; compile-time, so the forward carries none of it.
template <typename T, int HD, bool kSave = false>
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
  float* qraw;  // kSave only
  float* kraw;
  T* vrow;
  T* kt;

  // The bf16 kernel stages in LDS, after its main loop and for tiles holding q or k heads: the
  // multipliers 1 + w of the q and k norms (HD floats each), then for each of the tile's 256 rows
  // the RoPE (cos, sin) of pair p at float 2 HD + r kStgRow + 2p. Rows are padded to kStgRow floats
  // so that the 16 rows a quarter-wave reads fall in different banks. Reading the table from
  // global memory inside the epilogue, between its stores, made q and k tiles' epilogues several
  // times longer than the others'.
  static constexpr bool kStaged = true;
  static constexpr bool kLdsOut = false;
  static constexpr int kLdsOutFloats = 0;
  static constexpr bool kColumnHalves = true;  // for v and gate columns only (tail_allowed)
  // bf16, head_dim 128 (one head per wave): q, k and gate rows leave through a per-wave LDS area
  // placed after the staged tables, 16 rows at a time (rows of 256 bytes + 16 of padding), read
  // back 16 lanes per row so every store writes whole 256-byte rows (stored from the accumulator
  // layout, an instruction wrote 8 bytes into each of 32 rows). Measured at the 1024x1024 CFG pair
  // this gains under 1 % (1.427 -> 1.420 ms): the projection's remaining 6 % over a float32-output
  // GEMM of the same shape is not in its stores.
  static constexpr bool kOutStage = sizeof(T) == 2 && HD == 128;
  static constexpr int kOutPitch = 272;
  static constexpr int kOutFloats = kOutStage ? 16 * kOutPitch / 4 : 0;
  static constexpr int kStgRow = HD + 4;
  static constexpr int stage_floats() { return 2 * HD + 256 * kStgRow; }
  __device__ __forceinline__ bool wants_stage(int n0) const { return n0 < nq + nk; }
  // Run by the workgroup's 256 threads. Every table load is issued before the first LDS store, so
  // the staging costs one memory round trip (in batches of four loads per thread it took four).
  __device__ __forceinline__ void stage(float* st, int m0, int M, int tid) const {
    constexpr int NTHR = 256;
    constexpr int P4 = HD / 8;              // float4s of cos (or sin) per row: HD / 2 pairs
    constexpr int NI = 256 * P4 / NTHR;     // (cos, sin) float4 pairs per thread
    static_assert(256 * P4 % NTHR == 0 && 2 * HD <= 2 * NTHR, "staging split");
    float4 cv[NI], sv[NI];
    if (rc) {
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int i = tid + NTHR * k, r = i / P4, c4 = i - r * P4;
        const int m = m0 + r;
        const int l = (m < M ? m : 0) % L;
        cv[k] = ld4(rc + (size_t)l * (HD / 2) + 4 * c4);
        sv[k] = ld4(rs + (size_t)l * (HD / 2) + 4 * c4);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + NTHR * k;
      if (i < 2 * HD) {
        const float* w = i < HD ? wnq : wnk;
        st[i] = 1.0f + (w ? w[i % HD] : 0.0f);
      }
    }
    if (!rc) return;
    float* t = st + 2 * HD;
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int i = tid + NTHR * k, r = i / P4, c4 = i - r * P4;
      float* d = t + r * kStgRow + 8 * c4;
      st4(d, make_float4(cv[k].x, sv[k].x, cv[k].y, sv[k].y));
      st4(d + 4, make_float4(cv[k].z, sv[k].z, cv[k].w, sv[k].w));
    }
  }

  // q (seg 0), k (1) or gate (3) head of a wave through its output staging area (kOutStage). A q or
  // k tile always has its multipliers and (cos, sin) pairs staged in stg (wants_stage holds for every
  // tile that holds q or k columns), and whether RoPE applies is decided once, outside the unrolled
  // loops. With a test per group of four columns, and a global-memory path behind it, the compiler
  // waited for every memory operation in flight, the epilogue's own stores included, at each join
  // (198 full waits in the kernel).
  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply_staged(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                               int M, const float* stg, float* ostg, int seg) const {
    if (seg <= 1 && rc)
      apply_staged_t<LY, MI, NJ, true>(acc, row0, col0, lane, M, stg, ostg, seg);
    else
      apply_staged_t<LY, MI, NJ, false>(acc, row0, col0, lane, M, stg, ostg, seg);
  }

  template <class LY, int MI, int NJ, bool kRope>
  __device__ __forceinline__ void apply_staged_t(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                                 int M, const float* stg, float* ostg, int seg) const {
    T* const dst = seg == 0 ? q : seg == 1 ? k : g;
    const int ld = seg == 1 ? nk : nq;
    const int cb = seg == 0 ? col0 : seg == 1 ? col0 - nq : col0 - nq - 2 * nk;
    const float* const wst = stg + (seg == 0 ? 0 : HD);  // staged 1 + w of this head's norm
    char* const os = reinterpret_cast<char*>(ostg);
    const int r = lane & 31;                      // accumulator layout: row r, columns 32 jj + 8 qq + 4 (lane >> 5)
    const int rr = lane >> 4, ch = lane & 15;    // read-back: row 4 kk + rr, columns 8 ch .. 8 ch + 7
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = row0 + 32 * i + r;
      uint2 pk[NJ][4];
      if (seg <= 1) {
        float* const raw = seg == 0 ? qraw : kraw;
        if (kSave && m < M) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) st4(raw + (size_t)m * ld + cb + LY::col(jj, qq, lane), quad(acc[i][jj], qq));
        }
        float ss = 0.0f;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) ss += acc[i][jj][e] * acc[i][jj][e];
        ss = LY::rowsum(ss);
        const float inv = rsqrtf(ss * (1.0f / HD) + eps);
        const float* const cst = stg + 2 * HD + ((row0 & 255) + 32 * i + r) * kStgRow;  // this row's (cos, sin)
#pragma unroll
        for (int jq = 0; jq < 2 * NJ; ++jq) {
          // the LDS operands of two groups of four columns in one batch, so that one wait covers
          // them (read one group at a time, each read waited for its own latency: the output
          // staging's writes may alias them as far as the compiler can tell)
          const int jj = jq >> 1;
          float4 w4[2], cs[2];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            w4[x] = ld4(wst + LY::col(jj, 2 * (jq & 1) + x, lane));
            if constexpr (kRope) cs[x] = ld4(cst + LY::col(jj, 2 * (jq & 1) + x, lane));
          }
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int qq = 2 * (jq & 1) + x;
            const int d = LY::col(jj, qq, lane);
            float4 y = quad(acc[i][jj], qq);
            const float4 w = w4[x];
            y.x *= inv * w.x; y.y *= inv * w.y; y.z *= inv * w.z; y.w *= inv * w.w;
            if constexpr (kRope) {
              const float4 c = cs[x];
              y = make_float4(y.x * c.x - y.y * c.y, y.y * c.x + y.x * c.y,
                              y.z * c.z - y.w * c.w, y.w * c.z + y.z * c.w);
            }
            pk[jj][qq] = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
            if (kSave && seg == 1 && m < M) {  // k transposed per (batch, kv head), like vt
              const int b = m / L;
              T* kp = kt + (size_t)(b * (nk / HD) + cb / HD) * HD * ldvt + (m - b * L);
              const int dd = cb % HD + d;
              kp[(size_t)dd * ldvt] = to_t<T>(y.x);
              kp[(size_t)(dd + 1) * ldvt] = to_t<T>(y.y);
              kp[(size_t)(dd + 2) * ldvt] = to_t<T>(y.z);
              kp[(size_t)(dd + 3) * ldvt] = to_t<T>(y.w);
            }
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float4 y = quad(acc[i][jj], qq);
            pk[jj][qq] = make_uint2(pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w));
          }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {  // rows 16 hh .. 16 hh + 15 of the block
        if ((r >> 4) == hh) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              *reinterpret_cast<uint2*>(os + (r & 15) * kOutPitch + 2 * LY::col(jj, qq, lane)) = pk[jj][qq];
        }
        wave_lds_sync();  // the reads below see every lane's writes above
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = 4 * kk + rr;
          const uint4 v = *reinterpret_cast<const uint4*>(os + row * kOutPitch + 16 * ch);
          const int mm = row0 + 32 * i + 16 * hh + row;
          if (mm < M) *reinterpret_cast<uint4*>(dst + (size_t)mm * ld + cb + 8 * ch) = v;
        }
        wave_lds_sync();  // the next writes come after every lane's reads
      }
    }
  }

  template <class LY, int MI, int NJ>
  __device__ __forceinline__ void apply(const typename LY::F (&acc)[MI][NJ], int row0, int col0, int lane,
                                        int M, float* stg = nullptr, float* ostg = nullptr) const {
    constexpr int BS = LY::NQ == 1 ? 16 : 32;
    constexpr int HB = HD / BS;  // column blocks per head
    const int ntot = 2 * nq + 2 * nk;
    if constexpr (kOutStage && LY::NQ == 4 && NJ == HB) {
      if (col0 >= ntot) return;
      const int seg = col0 < nq ? 0 : col0 < nq + nk ? 1 : col0 < nq + 2 * nk ? 2 : 3;  // wave-uniform
      if (seg != 2) {
        apply_staged<LY, MI, NJ>(acc, row0, col0, lane, M, stg, ostg, seg);
        return;
      }
      // one v head, transposed per (batch, kv head); a path of its own so that the code for the
      // other segments, never taken here, does not weigh on this one
      const int vc0 = col0 - nq - nk;  // first column within v (a head boundary)
      const int kvh = vc0 / HD, nkvh = nk / HD;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int m = row0 + LY::row(i, lane);
        if (m >= M) continue;
        const int b = m / L, l = m - b * L;
        T* const base = vt + (size_t)(b * nkvh + kvh) * HD * ldvt + l;
        if constexpr (kSave) {
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int qq = 0; qq < LY::NQ; ++qq) st4(vrow + (size_t)m * nk + vc0 + LY::col(jj, qq, lane), quad(acc[i][jj], qq));
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
          for (int qq = 0; qq < LY::NQ; ++qq) {
            const int d = LY::col(jj, qq, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) base[(size_t)(d + e) * ldvt] = to_t<T>(acc[i][jj][4 * qq + e]);
          }
      }
      return;
    }
    if constexpr (NJ % HB != 0) {
      // A wave narrower than a head (the 256x128 halves of a last partial round): the host runs
      // such tiles only over v and gate columns (tail_allowed), which need no per-head reduction.
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int nb = col0 + j * BS;  // first column of this block (wave-uniform)
        if (nb >= ntot) break;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          const int m = row0 + LY::row(i, lane);
          if (m >= M) continue;
          if (nb < nq + 2 * nk) {
            const int b = m / L, l = m - b * L;
#pragma unroll
            for (int qq = 0; qq < LY::NQ; ++qq) {
              const int vc = col0 - nq - nk + LY::col(j, qq, lane);  // column within v
              if constexpr (kSave) st4(vrow + (size_t)m * nk + vc, quad(acc[i][j], qq));
              T* base = vt + (size_t)(b * (nk / HD) + vc / HD) * HD * ldvt + l;
#pragma unroll
              for (int e = 0; e < 4; ++e) base[(size_t)(vc % HD + e) * ldvt] = to_t<T>(acc[i][j][4 * qq + e]);
            }
          } else {
#pragma unroll
            for (int qq = 0; qq < LY::NQ; ++qq)
              st4(g + (size_t)m * nq + (col0 - nq - 2 * nk) + LY::col(j, qq, lane), quad(acc[i][j], qq));
          }
        }
      }
    } else {
#pragma unroll
      for (int h0 = 0; h0 < NJ; h0 += HB) {
        const int nh0 = col0 + h0 * BS;  // first column of this head (wave-uniform)
        if (nh0 >= ntot) break;
        const int seg = nh0 < nq ? 0 : nh0 < nq + nk ? 1 : nh0 < nq + 2 * nk ? 2 : 3;
        if (seg <= 1) {
          T* dst = seg == 0 ? q : k;
          const int ld = seg == 0 ? nq : nk;
          const int cb = seg == 0 ? nh0 : nh0 - nq;
          const float* wn = seg == 0 ? wnq : wnk;
          float* const raw = seg == 0 ? qraw : kraw;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int m = row0 + LY::row(i, lane);  // every lane sharing this row takes the same branches
            if (kSave && m < M) {
#pragma unroll
              for (int jj = 0; jj < HB; ++jj)
#pragma unroll
                for (int qq = 0; qq < LY::NQ; ++qq)
                  st4(raw + (size_t)m * ld + cb + LY::col(jj, qq, lane), quad(acc[i][h0 + jj], qq));
            }
            float ss = 0.0f;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj)
#pragma unroll
              for (int r = 0; r < 4 * LY::NQ; ++r) ss += acc[i][h0 + jj][r] * acc[i][h0 + jj][r];
            ss = LY::rowsum(ss);
            const float inv = rsqrtf(ss * (1.0f / HD) + eps);
            const int l = (m < M ? m : 0) % L;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj)
#pragma unroll
              for (int qq = 0; qq < LY::NQ; ++qq) {
                const int d = LY::col(jj, qq, lane);
                float4 y = quad(acc[i][h0 + jj], qq);
                if (stg) {  // staged multipliers and (cos, sin) pairs
                  const float4 w4 = ld4(stg + (seg == 0 ? 0 : HD) + d);
                  y.x *= inv * w4.x; y.y *= inv * w4.y; y.z *= inv * w4.z; y.w *= inv * w4.w;
                  if (rc) {
                    const float4 cs = ld4(stg + 2 * HD + ((row0 & 255) + LY::row(i, lane)) * kStgRow + d);
                    y = make_float4(y.x * cs.x - y.y * cs.y, y.y * cs.x + y.x * cs.y,
                                    y.z * cs.z - y.w * cs.w, y.w * cs.z + y.z * cs.w);
                  }
                } else {
                  const float4 w4 = wn ? ld4(wn + d) : make_float4(0.f, 0.f, 0.f, 0.f);
                  y.x *= inv * (1.0f + w4.x); y.y *= inv * (1.0f + w4.y);
                  y.z *= inv * (1.0f + w4.z); y.w *= inv * (1.0f + w4.w);
                  if (rc) {
                    const float2 c2 = *reinterpret_cast<const float2*>(rc + (size_t)l * (HD / 2) + (d >> 1));
                    const float2 s2 = *reinterpret_cast<const float2*>(rs + (size_t)l * (HD / 2) + (d >> 1));
                    y = make_float4(y.x * c2.x - y.y * s2.x, y.y * c2.x + y.x * s2.x,
                                    y.z * c2.y - y.w * s2.y, y.w * c2.y + y.z * s2.y);
                  }
                }
                if (m < M) {
                  st4(dst + (size_t)m * ld + cb + d, y);
                  if (kSave && seg == 1) {  // k transposed per (batch, kv head), like vt
                    const int b = m / L;
                    T* kp = kt + (size_t)(b * (nk / HD) + cb / HD) * HD * ldvt + (m - b * L);
                    const int dd = cb % HD + d;
                    kp[(size_t)dd * ldvt] = to_t<T>(y.x);
                    kp[(size_t)(dd + 1) * ldvt] = to_t<T>(y.y);
                    kp[(size_t)(dd + 2) * ldvt] = to_t<T>(y.z);
                    kp[(size_t)(dd + 3) * ldvt] = to_t<T>(y.w);
                  }
                }
              }
          }
        } else if (seg == 2) {
          const int kvh = (nh0 - nq - nk) / HD;
          const int nkvh = nk / HD;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int m = row0 + LY::row(i, lane);
            if (m >= M) continue;
            const int b = m / L, l = m - b * L;
            T* base = vt + (size_t)(b * nkvh + kvh) * HD * ldvt + l;
            if constexpr (kSave) {
#pragma unroll
              for (int jj = 0; jj < HB; ++jj)
#pragma unroll
                for (int qq = 0; qq < LY::NQ; ++qq)
                  st4(vrow + (size_t)m * nk + (nh0 - nq - nk) + LY::col(jj, qq, lane), quad(acc[i][h0 + jj], qq));
            }
#pragma unroll
            for (int jj = 0; jj < HB; ++jj)
#pragma unroll
              for (int qq = 0; qq < LY::NQ; ++qq) {
                const int d = LY::col(jj, qq, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) base[(size_t)(d + e) * ldvt] = to_t<T>(acc[i][h0 + jj][4 * qq + e]);
              }
          }
        } else {
          const int cb = nh0 - nq - 2 * nk;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int m = row0 + LY::row(i, lane);
            if (m >= M) continue;
#pragma unroll
            for (int jj = 0; jj < HB; ++jj)
#pragma unroll
              for (int qq = 0; qq < LY::NQ; ++qq)
                st4(g + (size_t)m * nq + cb + LY::col(jj, qq, lane), quad(acc[i][h0 + jj], qq));
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------------------------
// Tile order
// ---------------------------------------------------------------------------------------------

// ---------------------------------------------------------------------------------------------
// Main loop
// ---------------------------------------------------------------------------------------------

// 128-byte LDS rows, 32 consecutive rows read at 2 consecutive chunks (the 32x32x16 fragment
// pattern) and 8 rows x 8 chunks written at once: conflict-free on gfx950 (measured with the LDS
// bank-conflict counter).
__device__ __forceinline__ int swz128(int row) { return (row >> 1) & 7; }

template <typename T, int BM, int BN, int WM, int WN, class BMap, class Epi>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const T* __restrict__ A, int lda, int M, int K, int Ntot, int scn, BMap bmap, Epi epi) {
  constexpr int NWN = BN / WN, NW = (BM / WM) * NWN, NT = NW * 64;
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = 8;               // chunks per 128-byte LDS row
  constexpr int BK = CPR * EPC;        // bf16: 64, fp32: 32
  constexpr int FC = 8 / EPC;          // chunks per 8-element fragment
  constexpr int KS = BK / 32;          // 32-wide k chunks per slab
  constexpr int RSTEP = NT / CPR;      // rows moved by one load instruction of the workgroup
  constexpr int A_LD = BM / RSTEP, B_LD = BN / RSTEP;
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0 && 64 % RSTEP == 0, "tile/thread mismatch");
  // bf16 accumulates 32x32 blocks with v_mfma_f32_32x32x16_bf16 (about twice the rate of the
  // 16x16x32 form on this part); fp32 keeps 16x16 blocks.
  constexpr bool W32 = sizeof(T) == 2;
  constexpr int BS = W32 ? 32 : 16;
  constexpr int MI = WM / BS, NJ = WN / BS;
  typedef typename FragOf<T>::type Frag;
  typedef typename std::conditional<W32, f32x16, f32x4>::type Acc;
  auto swz = [](int row) { return W32 ? swz128(row) : swz8(row); };

  __shared__ uint4 smem[2][(BM + BN) * CPR];
  K2_LDS_CHECK(sizeof(smem), 1);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (Ntot + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, scn, tm, tn);
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
    a_dst[i] = row * CPR + (c ^ swz(row));
  }
  b_off = (uint32_t)(r * bmap.ldb + c * EPC) * sizeof(T);
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int row = r + i * RSTEP;
    b_dst[i] = (BM + row) * CPR + (c ^ swz(row));
  }

  Acc acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < (int)(sizeof(Acc) / 4); ++r) acc[i][j][r] = 0.0f;

  uint4 ra0[A_LD], rb0[B_LD], ra1[A_LD], rb1[B_LD];
  const int nk = (K + BK - 1) / BK;
  const int nk2 = (nk + 1) & ~1;  // slabs past K load zeros, so the loop runs in pairs of slabs

#define K2_GLOAD(RA, RB, kt)                                                                 \
  do {                                                                                       \
    const int k0_ = (kt) * BK;                                                               \
    const bool kin_ = k0_ + c * EPC < K;                                                     \
    const uint32_t kb_ = (uint32_t)k0_ * sizeof(T);                                          \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) RA[i] = bload(ra_src, kin_ ? a_off[i] + kb_ : kOOB); \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) RB[i] = bload(rb_src[i], kin_ ? b_off + kb_ : kOOB); \
    __builtin_amdgcn_sched_barrier(0); /* keep the loads ahead of the slab's matrix-core work */ \
  } while (0)

#define K2_SSTORE(RA, RB, buf)                                                \
  do {                                                                        \
    _Pragma("unroll") for (int i = 0; i < A_LD; ++i) smem[buf][a_dst[i]] = RA[i]; \
    _Pragma("unroll") for (int i = 0; i < B_LD; ++i) smem[buf][b_dst[i]] = RB[i]; \
  } while (0)

  // One slab from LDS stage `buf`. 32x32x16 (bf16): lane l supplies row/column l%32 and k slots
  // 8*(l/32)..+7 of a 16-wide k step, i.e. chunk 2s + l/32 of the 128-byte row for step s.
  // 16x16 (fp32): lane l supplies row/column l%16 and fragment chunks of lane group l/16.
#define K2_COMPUTE(buf)                                                                          \
  do {                                                                                           \
    const uint4* sA = smem[buf];                                                                 \
    const uint4* sB = smem[buf] + BM * CPR;                                                      \
    if constexpr (W32) {                                                                         \
      _Pragma("unroll") for (int s = 0; s < BK / 16; ++s) {                                      \
        bf16x8 fa[MI], fb[NJ];                                                                   \
        const int ch = 2 * s + (lane >> 5);                                                      \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
          const int row = wm * WM + i * 32 + (lane & 31);                                        \
          fa[i] = __builtin_bit_cast(bf16x8, sA[row * CPR + (ch ^ swz128(row))]);                \
        }                                                                                        \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                         \
          const int row = wn * WN + j * 32 + (lane & 31);                                        \
          fb[j] = __builtin_bit_cast(bf16x8, sB[row * CPR + (ch ^ swz128(row))]);                \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
          _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                         \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0); \
      }                                                                                          \
    } else {                                                                                     \
      _Pragma("unroll") for (int ks = 0; ks < KS; ++ks) {                                        \
        Frag af[MI], bfr[NJ];                                                                    \
        const int cb = ks * 4 * FC + (lane >> 4) * FC;                                           \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
          const int row = wm * WM + i * 16 + (lane & 15);                                        \
          _Pragma("unroll") for (int f = 0; f < FC; ++f)                                         \
            ((uint4*)&af[i])[f] = sA[row * CPR + ((cb + f) ^ swz8(row))];                        \
        }                                                                                        \
        _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                         \
          const int row = wn * WN + j * 16 + (lane & 15);                                        \
          _Pragma("unroll") for (int f = 0; f < FC; ++f)                                         \
            ((uint4*)&bfr[j])[f] = sB[row * CPR + ((cb + f) ^ swz8(row))];                       \
        }                                                                                        \
        _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
          _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i][j] = mma16(acc[i][j], bfr[j], af[i]); \
      }                                                                                          \
    }                                                                                            \
  } while (0)

  // Slab j is loaded into registers during step j-2 and written to LDS at the end of step j-1, so
  // its global loads have about two slabs of matrix-core work to land.
  K2_GLOAD(ra0, rb0, 0);
  K2_GLOAD(ra1, rb1, 1);
  K2_SSTORE(ra0, rb0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk2; kt += 2) {
    K2_GLOAD(ra0, rb0, kt + 2);  // LDS[0] holds slab kt; slab kt+1 is in flight in ra1/rb1
    K2_COMPUTE(0);
    K2_SSTORE(ra1, rb1, 1);
    __syncthreads();
    K2_GLOAD(ra1, rb1, kt + 3);  // LDS[1] holds slab kt+1; slab kt+2 is in flight in ra0/rb0
    K2_COMPUTE(1);
    K2_SSTORE(ra0, rb0, 0);
    __syncthreads();
  }
#undef K2_COMPUTE
#undef K2_GLOAD
#undef K2_SSTORE
  epi.template apply<Lay<BS>, MI, NJ>(acc, m0 + wm * WM, n0 + wn * WN, lane, M);
}

// ---------------------------------------------------------------------------------------------
// bf16 main loop: 256x256 workgroup tile, 4 waves (one per SIMD), each owning a 128x128 sub-tile
// of 4x4 blocks of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, in AGPRs).
//
// K advances in 64-wide slabs. A slab of A (256 rows) and a slab of W (256 rows) are LDS rows of
// one 128-byte line each, streamed by buffer->LDS DMA into two rings of 32 KB stages: RA stages for
// A, RB for W. An operand with R stages has its slab k+R fetched while slab k+1 is read, so its
// data has R-1 slabs of matrix-core time to arrive; 2 + 3 stages fill the 160 KB of LDS and the
// third stage goes to the operand whose data comes from furthest away. A DMA instruction moves
// 1 KB = 8 rows: lane i writes row i/8 at chunk position i%8, so it fetches global chunk (i%8) ^
// swz128(row), which is how the XOR swizzle is applied. Rows past M or past a weight matrix's end
// and chunks past K are out of the buffer's range and read as zero.
//
// Inside a slab the wave runs 4 k16 sub-steps of 16 matrix-core instructions; fragments are
// double-buffered in registers, each of the next sub-step's 8 fragment reads issued right after
// one of this sub-step's matrix-core instructions. The instruction order is spelled out and
// pinned with scheduling fences. One barrier per slab (a "turn"), before its last sub-step: by
// then every wave has read the slab's last fragments and has seen its own DMA of the next slab
// land, so the slab's two stages are refilled and the next slab's first fragments are read during
// the last sub-step. Stage addresses rotate at run time, so the loop body is one turn whatever the
// ring lengths. Loads complete in issue order, so within a turn the shorter ring's DMAs go first:
// the wait before the next slab's reads then leaves the deeper ring's newest DMAs in flight.
//
// SPREAD picks where the DMA instructions of a turn go. 0: all right after the barrier, which
// gives them the whole slab to land (best when the weights exceed the 256 MB last-level cache and
// come from HBM). 2 or 4: interleaved evenly with the matrix-core instructions of the first 2 or
// all 4 sub-steps after the barrier, which keeps them from stalling the wave in a burst (measured
// 10-15% faster than 0 when the operands stay cache-resident).
//
// KFULL (K a multiple of 64): every slab is whole, so a DMA's lane offsets are fixed and the slab's
// K offset goes in the instruction's scalar offset; slabs past K (fetched ahead, never read) reload
// slab 0. Otherwise each lane checks its chunk against K and chunks past it read as zero.
//
// MI_ and NJ pick the wave's M height (32 * MI_) and N width (32 * NJ): 4 and 4 give the 256x256
// tile; (4, 2) a 256x128 and (2, 4) a 128x256 half tile, used to split the last partial round of
// tiles so that it takes half as long (see gemm_bf16_kernel). A 128x256 half keeps the wave's full
// 128 columns, which the SwiGLU pairs and the per-head q/k norms need.
// ---------------------------------------------------------------------------------------------
template <int RA, int RB>
struct Rings {
  static_assert(RA >= 2 && RB >= 2 && (RA == 2 || RB == 2), "at most one ring is deeper than 2");
  static constexpr bool B_FIRST = RA > RB;  // DMA issue order within a turn: shorter ring first
  static constexpr int RMAX = RA > RB ? RA : RB, RMIN = RA < RB ? RA : RB;
  // 16-byte LDS units the rings need for a 256 x (64 NJ) tile
  static constexpr int units(int NJ) { return (RA * 256 + RB * 64 * NJ) * 8; }
};

template <int SPREAD, bool KFULL, int MI_, int NJ, int RA, int RB, class BMap, class Epi>
__device__ __forceinline__ void gemm_tile(const bf16* __restrict__ A, int lda, int M, int K, int Ntot, int m0, int n0,
                                          const BMap& bmap, const Epi& epi, uint4* lds) {
  typedef Rings<RA, RB> R;
  constexpr int BM = 64 * MI_, BN = 64 * NJ, WM = 32 * MI_, WN = 32 * NJ, BK = 64;
  constexpr int MI = MI_;
  constexpr int NRD = MI + NJ, NMF = MI * NJ;  // fragment reads / matrix-core ops per sub-step
  constexpr int NBA = BM / 32, NBB = BN / 32;  // 1 KB DMA blocks (8 rows) per wave per slab: A, B
  constexpr int DPW = NBA + NBB;               // DMA instructions per wave per slab
  constexpr int SA = BM * 8, SB = BN * 8;      // stage sizes in 16-byte units
  // DMAs a wait before a slab's reads may leave in flight: the deeper ring's of the last turn
  constexpr int NDEEP = RA == RB ? 0 : (R::B_FIRST ? NBA : NBB);
  // ... and before slab 0: those of the prologue issued after both rings' slab 0
  constexpr int W0 = NDEEP + DPW * (R::RMIN - 1);
  static_assert(W0 < 64, "vmcnt range");
  uint4* const ringA = lds;
  uint4* const ringB = lds + RA * SA;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: resources live in SGPRs
  const int wm = wave >> 1, wn = wave & 1;

  // DMA duties: wave w moves A rows 8*NBA*w .. and B rows 8*NBB*w .. of the tile, in blocks of
  // 8 rows. Block j's rows are 8j .. 8j+7 past the wave's first row; swz128 of its rows depends only
  // on j's parity, so two chunk choices cover all blocks.
  const int pos = lane & 7, lr = lane >> 3;
  const int cc[2] = {pos ^ ((lr >> 1) & 7), pos ^ ((4 + (lr >> 1)) & 7)};
  const rsrc_t ra = make_rsrc(A + (size_t)m0 * lda, (size_t)(M - m0) * lda * sizeof(bf16));
  uint32_t avo[2], bvo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    avo[p] = (uint32_t)((8 * NBA * wave + lr) * lda + cc[p] * 8) * sizeof(bf16);
    bvo[p] = (uint32_t)(lr * bmap.ldb + cc[p] * 8) * sizeof(bf16);
  }
  const uint32_t arow8 = (uint32_t)(8 * lda) * sizeof(bf16);  // byte distance of consecutive A blocks
  rsrc_t rb[NBB];
#pragma unroll
  for (int j = 0; j < NBB; ++j) {
    const int n = n0 + 8 * NBB * wave + 8 * j;
    int nvalid = 0;
    const bf16* base = n < Ntot ? bmap.group(n, nvalid) : A;
    nvalid = n < Ntot ? (nvalid < 0 ? 0 : (nvalid > 8 ? 8 : nvalid)) : 0;
    rb[j] = make_rsrc(base, (size_t)nvalid * bmap.ldb * sizeof(bf16));
  }
  // DMA block j of A slab kt into A stage ST, of B slab kt into B stage ST
#define K2_DMA_A(ST, kt, j)                                                                      \
  do {                                                                                           \
    const int k0_ = (kt) * BK;                                                                   \
    if (KFULL)                                                                                   \
      dma16(ra, (ST) + (8 * NBA * wave + 8 * (j)) * 8, avo[(j) & 1] + (j) * arow8,                    \
            (uint32_t)(k0_ < K ? k0_ : 0) * sizeof(bf16));                                       \
    else                                                                                         \
      dma16(ra, (ST) + (8 * NBA * wave + 8 * (j)) * 8,                                                \
            k0_ + cc[(j) & 1] * 8 < K ? avo[(j) & 1] + (j) * arow8 + (uint32_t)k0_ * sizeof(bf16) : kOOB, 0); \
  } while (0)
#define K2_DMA_B(ST, kt, j)                                                                      \
  do {                                                                                           \
    const int k0_ = (kt) * BK;                                                                   \
    if (KFULL)                                                                                   \
      dma16(rb[j], (ST) + (8 * NBB * wave + 8 * (j)) * 8, bvo[(j) & 1],                          \
            (uint32_t)(k0_ < K ? k0_ : 0) * sizeof(bf16));                                       \
    else                                                                                         \
      dma16(rb[j], (ST) + (8 * NBB * wave + 8 * (j)) * 8,                                        \
            k0_ + cc[(j) & 1] * 8 < K ? bvo[(j) & 1] + (uint32_t)k0_ * sizeof(bf16) : kOOB, 0);  \
  } while (0)
  // DMA instruction d (0 .. DPW-1) of a turn: A slab kA into STA, B slab kB into STB, shorter ring first
#define K2_DMA1(d, STA, kA, STB, kB)                                                             \
  do {                                                                                           \
    if (R::B_FIRST) {                                                                            \
      if ((d) < NBB) K2_DMA_B(STB, kB, (d) % NBB);                                               \
      else K2_DMA_A(STA, kA, ((d) - NBB) % NBA);                                                 \
    } else {                                                                                     \
      if ((d) < NBA) K2_DMA_A(STA, kA, (d) % NBA);                                               \
      else K2_DMA_B(STB, kB, ((d) - NBA) % NBB);                                                 \
    }                                                                                            \
  } while (0)

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment reads: lane l supplies row/column l%32 and k slots 8*(l/32)..+7 of a k16 sub-step,
  // i.e. chunk 2s + l/32 of the 128-byte row. The rows a lane reads all have the same swz128.
  const int fsw = ((lane & 31) >> 1) & 7, hh = lane >> 5;
  const int arow = (wm * WM + (lane & 31)) * 8, brow = (wn * WN + (lane & 31)) * 8;
  bf16x8 fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
#define K2_FENCE() __builtin_amdgcn_sched_barrier(0)
  // fragment q of sub-step s from stages (SA_, SB_): A blocks 0..MI-1, then B blocks 0..NJ-1
#define K2_READ1(FA, FB, SA_, SB_, s, q)                                                         \
  do {                                                                                           \
    const int ch_ = (2 * (s) + hh) ^ fsw;                                                        \
    if ((q) < MI) FA[(q) % MI] = __builtin_bit_cast(bf16x8, (SA_)[arow + ((q) % MI) * 256 + ch_]); \
    else FB[((q) - MI) % NJ] = __builtin_bit_cast(bf16x8, (SB_)[brow + (((q) - MI) % NJ) * 256 + ch_]); \
  } while (0)
  // one sub-step: the matrix-core work of (FA, FB); after instruction q, fragment q of sub-step RS
  // of stages (RSA, RSB) into (GA, GB) (q < NRD, RS >= 0) and DMA instructions D0 + [ceil(q ND /
  // NMF), ceil((q+1) ND / NMF)) of the turn (ND spread evenly over the NMF instructions)
#define K2_STEP(FA, FB, GA, GB, RSA, RSB, RS, D0, ND)                                            \
  do {                                                                                           \
    _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                                            \
      acc[q / NJ][q % NJ] =                                                                      \
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(FB[q % NJ], FA[q / NJ], acc[q / NJ][q % NJ], 0, 0, 0); \
      if ((RS) >= 0 && q < NRD) K2_READ1(GA, GB, RSA, RSB, RS, q);                               \
      _Pragma("unroll") for (int d_ = (q * (ND) + NMF - 1) / NMF; d_ < ((q + 1) * (ND) + NMF - 1) / NMF; ++d_) \
        K2_DMA1((D0) + d_, wA, kt + RA, wB, kt + RB);                                            \
      K2_FENCE();                                                                                \
    }                                                                                            \
  } while (0)
#define K2_BARRIER()                   \
  do {                                 \
    asm volatile("" ::: "memory");     \
    K2_FENCE();                        \
    __builtin_amdgcn_s_barrier();      \
    K2_FENCE();                        \
    asm volatile("" ::: "memory");     \
  } while (0)

  // Prologue: the DMAs turns -RMAX .. -1 would have issued (slabs 0 .. RA-1 of A, 0 .. RB-1 of B),
  // in turn order, then slab 0's first three sub-steps.
#pragma unroll
  for (int t = -R::RMAX; t < 0; ++t) {
    const int ja = t + RA, jb = t + RB;
    if (R::B_FIRST && jb >= 0) {
#pragma unroll
      for (int j = 0; j < NBB; ++j) K2_DMA_B(ringB + (jb % RB) * SB, jb, j);
    }
    if (ja >= 0) {
#pragma unroll
      for (int j = 0; j < NBA; ++j) K2_DMA_A(ringA + (ja % RA) * SA, ja, j);
    }
    if (!R::B_FIRST && jb >= 0) {
#pragma unroll
      for (int j = 0; j < NBB; ++j) K2_DMA_B(ringB + (jb % RB) * SB, jb, j);
    }
  }
  K2_WAIT_VM(W0);  // this wave's DMAs of slab 0 landed
  K2_BARRIER();
  {
    const int kt = 0;  // (no DMA in these steps)
    uint4* const wA = ringA;
    uint4* const wB = ringB;
#pragma unroll
    for (int q = 0; q < NRD; ++q) K2_READ1(fa0, fb0, ringA, ringB, 0, q);
    K2_STEP(fa0, fb0, fa1, fb1, ringA, ringB, 1, 0, 0);
    K2_STEP(fa1, fb1, fa0, fb0, ringA, ringB, 2, 0, 0);
    K2_STEP(fa0, fb0, fa1, fb1, ringA, ringB, 3, 0, 0);
  }
  // Turn kt: wait for slab kt+1, refill slab kt's stages (A with slab kt+RA, B with kt+RB), finish
  // slab kt and run sub-steps 0..2 of slab kt+1.
  // DMA instructions of a turn: step i of the SPREAD first steps issues [DS(i), DS(i+1))
  constexpr int NS = SPREAD > 0 ? SPREAD : 1;
#define K2_DS(i) ((i) < NS ? (i) * DPW / NS : DPW)
#define K2_DN(i) (SPREAD > 0 ? K2_DS((i) + 1) - K2_DS(i) : 0)
  const int nk = (K + BK - 1) / BK;
  int sa = 0, sb = 0;  // ring stages of slab kt
  for (int kt = 0; kt < nk - 1; ++kt) {
    const int sa1 = sa + 1 == RA ? 0 : sa + 1, sb1 = sb + 1 == RB ? 0 : sb + 1;
    uint4* const wA = ringA + sa * SA;
    uint4* const wB = ringB + sb * SB;
    const uint4* const rA = ringA + sa1 * SA;
    const uint4* const rB = ringB + sb1 * SB;
    K2_WAIT_VM(NDEEP);
    K2_WAIT_LGKM0();  // every read of slab kt has landed
    K2_BARRIER();
    if (SPREAD == 0) {
#pragma unroll
      for (int d = 0; d < DPW; ++d) K2_DMA1(d, wA, kt + RA, wB, kt + RB);
      K2_FENCE();
    }
    K2_STEP(fa1, fb1, fa0, fb0, rA, rB, 0, K2_DS(0), K2_DN(0));
    K2_STEP(fa0, fb0, fa1, fb1, rA, rB, 1, K2_DS(1), K2_DN(1));
    K2_STEP(fa1, fb1, fa0, fb0, rA, rB, 2, K2_DS(2), K2_DN(2));
    K2_STEP(fa0, fb0, fa1, fb1, rA, rB, 3, K2_DS(3), K2_DN(3));
    sa = sa1;
    sb = sb1;
  }
  K2_WAIT_LGKM0();
  {
    const int kt = 0;
    uint4* const wA = ringA;
    uint4* const wB = ringB;
    K2_STEP(fa1, fb1, fa0, fb0, ringA, ringB, -1, 0, 0);  // last sub-step of slab nk - 1
  }
  K2_WAIT_VM(0);  // no DMA may still write LDS when the workgroup retires
  float* stg = nullptr;
  if constexpr (Epi::kLdsOut) {
    static_assert(4 * Epi::kLdsOutFloats * sizeof(float) <= Rings<RA, RB>::units(4) * sizeof(uint4), "LDS output");
    __syncthreads();  // every wave is done with the rings
    stg = reinterpret_cast<float*>(lds) + wave * Epi::kLdsOutFloats;
  }
  if constexpr (Epi::kStaged) {
    static_assert(Epi::stage_floats() * sizeof(float) <= Rings<RA, RB>::units(4) * sizeof(uint4), "LDS staging");
    if (epi.wants_stage(n0)) {  // tile-uniform
      __syncthreads();  // every wave is done with the rings
      epi.stage(reinterpret_cast<float*>(lds), m0 & ~255, M, tid);  // 256 threads; the whole 256-row tile's rows
      __syncthreads();
      stg = reinterpret_cast<float*>(lds);
    }
  }
#undef K2_DN
#undef K2_DS
#undef K2_BARRIER
#undef K2_STEP
#undef K2_READ1
#undef K2_FENCE
#undef K2_DMA1
#undef K2_DMA_B
#undef K2_DMA_A
  if constexpr (Epi::kOutStage) {
    static_assert((Epi::stage_floats() + 4 * Epi::kOutFloats) * sizeof(float) <= Rings<RA, RB>::units(4) * sizeof(uint4),
                  "LDS output staging");
    if (!stg) __syncthreads();  // every wave is done with the rings (the staging branch synced already)
    float* const ostg = reinterpret_cast<float*>(lds) + Epi::stage_floats() + wave * Epi::kOutFloats;
    epi.template apply<Lay<32>, MI, NJ>(acc, m0 + wm * WM, n0 + wn * WN, lane, M, stg, ostg);
  } else {
    epi.template apply<Lay<32>, MI, NJ>(acc, m0 + wm * WM, n0 + wn * WN, lane, M, stg);
  }
}

// Workgroups 0 .. nmain-1 each compute a 256x256 tile (tile order: tile_coords). With TAIL, the
// tiles_total - nmain tiles of the last partial round (or all tiles, nmain = 0, when they fill at
// most half a round) are split in two halves run by workgroups nmain + 2u and nmain + 2u + 1 (u:
// tail tile index), so that round takes about half as long; TAIL is used when the halves fit in
// one round. TAIL 1: 256x128 halves (column halves); TAIL 2: 128x256 halves (row halves), for the
// epilogues that need a wave's full 128 columns (SwiGLU; q and k heads). TAIL 0: no halves.
template <int SPREAD, bool KFULL, int RA, int RB, int TAIL, class BMap, class Epi>
__global__ void __launch_bounds__(256)
gemm_bf16_kernel(const bf16* __restrict__ A, int lda, int M, int K, int Ntot, int scn, int nmain, BMap bmap,
                 Epi epi) {
  __shared__ uint4 lds[Rings<RA, RB>::units(4)];
  K2_LDS_CHECK(sizeof(lds), 1);
  const int tiles_m = (M + 255) / 256, tiles_n = (Ntot + 255) / 256;
  const int bid = blockIdx.x;
  int tm, tn;
  if (TAIL == 0 || bid < nmain) {
    tile_coords(bid, tiles_m, tiles_n, scn, tm, tn);
    gemm_tile<SPREAD, KFULL, 4, 4, RA, RB>(A, lda, M, K, Ntot, tm * 256, tn * 256, bmap, epi, lds);
  } else if constexpr (TAIL == 2) {
    const int u = bid - nmain;
    tile_coords(nmain + (u >> 1), tiles_m, tiles_n, scn, tm, tn);
    const int m0 = tm * 256 + (u & 1) * 128;
    if (m0 >= M) return;  // the second half of a last M-tile of at most 128 rows (workgroup-uniform)
    gemm_tile<SPREAD, KFULL, 2, 4, RA, RB>(A, lda, M, K, Ntot, m0, tn * 256, bmap, epi, lds);
  } else if constexpr (TAIL == 1 && Epi::kColumnHalves) {
    const int u = bid - nmain;
    tile_coords(nmain + (u >> 1), tiles_m, tiles_n, scn, tm, tn);
    gemm_tile<SPREAD, KFULL, 4, 2, RA, RB>(A, lda, M, K, Ntot, tm * 256, tn * 256 + (u & 1) * 128, bmap, epi, lds);
  }
}

// ---------------------------------------------------------------------------------------------
// Launch configurations
// ---------------------------------------------------------------------------------------------
template <typename T> struct Cfg;
template <> struct Cfg<bf16> {
  static constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
  static constexpr bool DMA = true;
};
template <> struct Cfg<float> { static constexpr int BM = 64, BN = 128, WM = 32, WN = 128; static constexpr bool DMA = false; };

// Compute units of the current device (one bf16 GEMM workgroup runs per compute unit).
static int compute_units() {
  static thread_local int dev_cached = -1, cu_cached = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev != dev_cached) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    dev_cached = dev;
    cu_cached = n;
  }
  return cu_cached;
}

// LDS ring depths of the bf16 kernel: the third stage goes to the weights. Measured on the block's
// shapes against 2 + 2 (the same instruction stream): SwiGLU up 8 %, down projection 6 %, output
// projection unchanged; 3 + 2 loses on SwiGLU. The weights' slabs are the ones that arrive late:
// each super-column starts on weight rows that are still in HBM.
constexpr int kRingA = 2, kRingB = 3;

// Whether the 256x128 halves of a last partial round may start at column n0 (every epilogue but
// the QKV+gate one takes any column; that one takes only v and gate columns in narrow waves).
template <class Epi>
static bool tail_allowed(const Epi&, int) { return Epi::kColumnHalves; }
template <typename T, int HD, bool kSave>
static bool tail_allowed(const EpiQkvg<T, HD, kSave>& e, int n0) { return n0 >= e.nq + e.nk; }
// TAIL: the last partial round may run as half tiles; ROWS: row halves are built for this
// configuration too (the one every model shape takes: K a multiple of 64, cache-resident weights).
template <typename T, class C, class BMap, class Epi, int SPREAD, bool KFULL, bool TAIL, bool ROWS = false>
static hipError_t launch_cfg(const GemmA& a, int Ntot, int scn, const BMap& bmap, const Epi& epi, hipStream_t s) {
  constexpr int NT = (C::BM / C::WM) * (C::BN / C::WN) * 64;
  const int tiles = ((a.M + C::BM - 1) / C::BM) * ((Ntot + C::BN - 1) / C::BN);
  if constexpr (sizeof(T) == 2 && C::DMA) {
    int nmain = tiles, grid = tiles, mrows = 0;
    if constexpr (TAIL) {
      // Half tiles where a round is partly idle: the last partial round when it holds at most half
      // the compute units, or every tile when all of them fill at most half a round (small M: the
      // 512^2 block's out and down projections are 120 tiles for 256 compute units).
      const int ncu = compute_units();
      const int tail = 2 * tiles <= ncu ? tiles : tiles % ncu;
      if (tail > 0 && 2 * tail <= ncu) {
        // column halves (measured on the block's shapes) where every tail tile's epilogue takes
        // them, row halves otherwise
        const int tiles_m = (a.M + 255) / 256, tiles_n = (Ntot + 255) / 256;
        bool cols = true;
        for (int u = tiles - tail; cols && u < tiles; ++u) {
          int tm, tn;
          tile_coords(u, tiles_m, tiles_n, scn, tm, tn);
          cols = tail_allowed(epi, tn * 256);
        }
        if (cols || ROWS) {
          mrows = cols ? 0 : 1;
          nmain = tiles - tail;
          grid = nmain + 2 * tail;
        }
      }
    }
    if (!TAIL || !mrows)
      hipLaunchKernelGGL((gemm_bf16_kernel<SPREAD, KFULL, kRingA, kRingB, TAIL ? 1 : 0, BMap, Epi>), dim3(grid),
                         dim3(256), 0, s, (const bf16*)a.A, a.lda, a.M, a.K, Ntot, scn, nmain, bmap, epi);
    else if constexpr (ROWS)
      hipLaunchKernelGGL((gemm_bf16_kernel<SPREAD, KFULL, kRingA, kRingB, 2, BMap, Epi>), dim3(grid), dim3(256), 0, s,
                         (const bf16*)a.A, a.lda, a.M, a.K, Ntot, scn, nmain, bmap, epi);
  } else {
    hipLaunchKernelGGL((gemm_kernel<T, C::BM, C::BN, C::WM, C::WN, BMap, Epi>), dim3(tiles), dim3(NT), 0, s,
                       (const T*)a.A, a.lda, a.M, a.K, Ntot, scn, bmap, epi);
  }
  return hipGetLastError();
}

// Launch policy, from measurements on the block's GEMM shapes:
//  - tile order: super-columns (see tile_coords) when the weights are the larger operand; when the
//    activations are larger, their re-reads per super-column cost more than they save;
//  - bf16 DMA schedule: spread among the matrix-core instructions (over SPREAD_CACHED sub-steps:
//    the SwiGLU projection runs best with 2, the other projections with 4), unless the weight rows
//    in use at once exceed the 256 MB last-level cache, in which case their slabs come from HBM
//    and need the whole slab period to land (DMA right after the barrier);
//  - K a multiple of 64 takes the scalar-offset DMA (2-5 % faster than per-lane K checks).
constexpr size_t kLastLevelCacheBytes = size_t(256) << 20;

template <typename T, class BMap, class Epi, bool TAIL = false, int SPREAD_CACHED = 4>
static hipError_t launch(const GemmA& a, int Ntot, const BMap& bmap, const Epi& epi, hipStream_t s) {
  typedef Cfg<T> C;
  if (a.M <= 0 || Ntot <= 0) return hipSuccess;
  const int tiles_n = (Ntot + C::BN - 1) / C::BN;
  const size_t a_bytes = (size_t)a.M * a.K * sizeof(T), b_bytes = (size_t)Ntot * a.K * sizeof(T);
  const int scn = b_bytes >= a_bytes ? super_cols(tiles_n, C::BN, a.K, sizeof(T)) : tiles_n;
  if constexpr (sizeof(T) == 2) {
    if (a.K % 64 != 0) return launch_cfg<T, C, BMap, Epi, 2, false, TAIL>(a, Ntot, scn, bmap, epi, s);
    if ((size_t)scn * C::BN * a.K * sizeof(T) > kLastLevelCacheBytes)
      return launch_cfg<T, C, BMap, Epi, 0, true, TAIL>(a, Ntot, scn, bmap, epi, s);
    return launch_cfg<T, C, BMap, Epi, SPREAD_CACHED, true, TAIL, TAIL>(a, Ntot, scn, bmap, epi, s);
  } else {
    return launch_cfg<T, C, BMap, Epi, 0, false, TAIL>(a, Ntot, scn, bmap, epi, s);
  }
}

template <typename T, int HD, bool kSave>
static hipError_t qkvg_t(const GemmA& a, const QkvgArgs& p, hipStream_t s) {
  BSegs<T> bm;
  bm.p[0] = (const T*)p.wq; bm.p[1] = (const T*)p.wk; bm.p[2] = (const T*)p.wv; bm.p[3] = (const T*)p.wg;
  bm.start[0] = 0; bm.start[1] = p.nq; bm.start[2] = p.nq + p.nk; bm.start[3] = p.nq + 2 * p.nk;
  bm.start[4] = 2 * p.nq + 2 * p.nk;
  bm.nseg = 4;
  bm.ldb = a.K;
  EpiQkvg<T, HD, kSave> e;
  e.q = (T*)p.q; e.k = (T*)p.k; e.vt = (T*)p.vt; e.g = (T*)p.g;
  e.wnq = p.wnq; e.wnk = p.wnk; e.rc = p.rope_cos; e.rs = p.rope_sin;
  e.nq = p.nq; e.nk = p.nk; e.L = p.L; e.ldvt = p.ldvt; e.eps = p.eps;
  e.qraw = p.qraw; e.kraw = p.kraw; e.vrow = (T*)p.vrow; e.kt = (T*)p.kt;
  return launch<T, BSegs<T>, EpiQkvg<T, HD, kSave>, true>(a, 2 * p.nq + 2 * p.nk, bm, e, s);
}

template <typename T, bool kSave>
static hipError_t swiglu_t(const GemmA& a, const SwigluArgs& p, hipStream_t s) {
  constexpr int WN = Cfg<T>::WN;
  constexpr int RSTEP = (Cfg<T>::BM / Cfg<T>::WM) * (Cfg<T>::BN / Cfg<T>::WN) * 64 / 8;
  static_assert((WN / 2) % RSTEP == 0, "a load group must not straddle gate and up rows");
  BSwiglu<T, WN> bm;
  bm.gate = (const T*)p.wgate; bm.up = (const T*)p.wup; bm.I = p.I; bm.ldb = a.K;
  EpiSwiglu<T, WN, kSave> e;
  e.a = (T*)p.a; e.I = p.I; e.gsave = p.gsave; e.usave = p.usave;
  const int ntot = ((p.I + WN / 2 - 1) / (WN / 2)) * WN;
  return launch<T, BSwiglu<T, WN>, EpiSwiglu<T, WN, kSave>, true, 2>(a, ntot, bm, e, s);
}

template <typename T>
static hipError_t resid_t(const GemmA& a, const ResidArgs& p, hipStream_t s) {
  BSegs<T> bm = {};
  bm.p[0] = (const T*)p.w; bm.start[0] = 0; bm.start[1] = p.N; bm.nseg = 1; bm.ldb = a.K;
  if (p.L >= 128) {  // a wave's 128 rows span at most two batch rows
    EpiResid<T, true> e;
    e.hin = p.hin; e.hout = p.hout; e.gate = p.gate; e.gate_stride = p.gate_stride; e.L = p.L; e.N = p.N;
    return launch<T, BSegs<T>, EpiResid<T, true>, true>(a, p.N, bm, e, s);
  }
  EpiResid<T, false> e;
  e.hin = p.hin; e.hout = p.hout; e.gate = p.gate; e.gate_stride = p.gate_stride; e.L = p.L; e.N = p.N;
  return launch<T, BSegs<T>, EpiResid<T, false>, true>(a, p.N, bm, e, s);
}

template <typename T>
static hipError_t plain_t(const GemmA& a, const PlainArgs& p, hipStream_t s) {
  BSegs<T> bm = {};
  bm.p[0] = (const T*)p.w; bm.start[0] = 0; bm.start[1] = p.N; bm.nseg = 1; bm.ldb = a.K;
  if (p.outf && !p.outt && !p.bias && p.out_rows_per_b == p.rows_per_b && p.out_row_off == 0 && p.N % 4 == 0 &&
      p.ldf % 4 == 0) {  // float32 output only, row m to row m
    EpiPlainF32<T> e;
    e.outf = p.outf; e.ldf = p.ldf; e.N = p.N;
    return launch<T, BSegs<T>, EpiPlainF32<T>, true>(a, p.N, bm, e, s);
  }
  EpiPlain<T> e;
  e.bias = p.bias; e.outf = p.outf; e.ldf = p.ldf; e.outt = (T*)p.outt; e.ldt = p.ldt; e.act = p.act;
  e.N = p.N; e.rpb = p.rows_per_b; e.orpb = p.out_rows_per_b; e.ooff = p.out_row_off;
  return launch<T, BSegs<T>, EpiPlain<T>, true>(a, p.N, bm, e, s);
}

template <bool kSave>
static hipError_t qkvg_d(int dt, const GemmA& a, const QkvgArgs& p, hipStream_t s) {
  if (p.hd == 128) return dt == DT_BF16 ? qkvg_t<bf16, 128, kSave>(a, p, s) : qkvg_t<float, 128, kSave>(a, p, s);
  if (p.hd == 64) return dt == DT_BF16 ? qkvg_t<bf16, 64, kSave>(a, p, s) : qkvg_t<float, 64, kSave>(a, p, s);
  return hipErrorInvalidValue;
}
// The saving variants run when all their outputs are given, the plain ones when none is.
hipError_t gemm_qkvg(int dt, const GemmA& a, const QkvgArgs& p, hipStream_t s) {
  const int n = !!p.qraw + !!p.kraw + !!p.vrow + !!p.kt;
  if (n == 0) return qkvg_d<false>(dt, a, p, s);
  if (n == 4) return qkvg_d<true>(dt, a, p, s);
  return hipErrorInvalidValue;
}
hipError_t gemm_swiglu(int dt, const GemmA& a, const SwigluArgs& p, hipStream_t s) {
  if (!p.gsave != !p.usave) return hipErrorInvalidValue;
  if (p.gsave) return dt == DT_BF16 ? swiglu_t<bf16, true>(a, p, s) : swiglu_t<float, true>(a, p, s);
  return dt == DT_BF16 ? swiglu_t<bf16, false>(a, p, s) : swiglu_t<float, false>(a, p, s);
}
hipError_t gemm_resid(int dt, const GemmA& a, const ResidArgs& p, hipStream_t s) {
  return dt == DT_BF16 ? resid_t<bf16>(a, p, s) : resid_t<float>(a, p, s);
}
hipError_t gemm_plain(int dt, const GemmA& a, const PlainArgs& p, hipStream_t s) {
  return dt == DT_BF16 ? plain_t<bf16>(a, p, s) : plain_t<float>(a, p, s);
}

}  // namespace k2
