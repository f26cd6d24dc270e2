// Bandwidth-bound kernels of the block and backbone (gfx950).
//
//   modnorm        — (1 + scale_b) * RMSNorm(h; w) + shift_b, float32 statistics, one workgroup per two
//                    rows, float4 loads and one pass over HBM (the rows stay in registers between the
//                    reduction and the write). Architecture article §四.2 (modulated pre-norms),
//                    §四.4 (zero-centred RMSNorm computed in float32), §四.6 (final-layer norm).
//   modulation     — temb chunks + per-block (6, H) table ([ARTICLE] §四.2), or e + (2, H) table for the
//                    final layer (§四.6).
//   rope_table     — cos/sin of the 3-axis rotary angles, once per forward ([ARTICLE] §四 data flow).
//   time_embed     — cos-first sinusoid of 1000 t ([ARTICLE] §四.5).
//   layer_compress — Linear(num_layers, 1, bias=False) over the text layer axis ([ARTICLE] §四.1).
//   to_f32/from_f32 — operand dtype conversions.
//   block_reach    — per-token reach of the block-causal attention (QwenImage 2.1 model page,
//                    block-causal attention item): the last position a query may attend.
#include "k2_device.h"
#include "k2_kernels.h"

#include <climits>

namespace k2 {

template <typename TO> __device__ __forceinline__ void store4(TO* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
  *(bf16x4*)p = v;
}

// R rows per workgroup, each held in registers between the reduction and the write; the weight
// and modulation vectors are read once for all R rows (two rows: 77 against 83 us at 9216 x 6144;
// three or four rows were slower).
template <typename TO, int R>
__global__ void __launch_bounds__(256) modnorm_kernel(ModnormArgs p) {
  constexpr int CACHE = 8;  // float4 per thread and row kept in registers (rows up to 8192 wide)
  __shared__ float red[R][4];
  K2_LDS_CHECK(sizeof(red), 1);
  const int r0 = R * blockIdx.x;
  const int nr = min(R, p.rows - r0);
  const int H4 = p.H >> 2;
  const float4* x[R];
  TO* y[R];
  int bb[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int r = k < nr ? r0 + k : r0;
    const int b = r / p.rows_per_b, i = r - b * p.rows_per_b;
    bb[k] = b;
    x[k] = (const float4*)(p.in + ((size_t)b * p.in_rows_per_b + p.in_row_off + i) * p.H);
    y[k] = (TO*)p.out + (size_t)r * p.H;
  }
  float4 v[R][CACHE];
  float ss[R];
#pragma unroll
  for (int k = 0; k < R; ++k) ss[k] = 0.0f;
#pragma unroll
  for (int u = 0; u < CACHE; ++u) {
    const int c = threadIdx.x + u * 256;
    if (c < H4) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        v[k][u] = x[k][c];
        ss[k] += v[k][u].x * v[k][u].x + v[k][u].y * v[k][u].y + v[k][u].z * v[k][u].z + v[k][u].w * v[k][u].w;
      }
    }
  }
  for (int c = threadIdx.x + CACHE * 256; c < H4; c += 256)
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float4 t = x[k][c];
      ss[k] += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
    }
#pragma unroll
  for (int k = 0; k < R; ++k) ss[k] = wave_sum(ss[k]);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) red[k][wv] = ss[k];
  }
  __syncthreads();
  float inv[R];
#pragma unroll
  for (int k = 0; k < R; ++k)
    inv[k] = rsqrtf((red[k][0] + red[k][1] + red[k][2] + red[k][3]) / (float)p.H + p.eps);
  const float4* w4 = (const float4*)p.w;
  const float* scb[R];
  const float* shb[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    scb[k] = p.scale ? p.scale + (size_t)bb[k] * p.mod_stride : nullptr;
    shb[k] = p.shift ? p.shift + (size_t)bb[k] * p.mod_stride : nullptr;
  }
  auto emit = [&](int c, const float4 (&t)[R]) {
    const float4 w = w4 ? w4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 sc = make_float4(0.f, 0.f, 0.f, 0.f), sh = sc;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (k >= nr) break;
      if (k == 0 || bb[k] != bb[k - 1]) {  // a new batch row: its modulation vectors
        sc = scb[k] ? ((const float4*)scb[k])[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        sh = shb[k] ? ((const float4*)shb[k])[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      store4<TO>(y[k] + 4 * c, (1.0f + sc.x) * (t[k].x * inv[k] * (1.0f + w.x)) + sh.x,
                 (1.0f + sc.y) * (t[k].y * inv[k] * (1.0f + w.y)) + sh.y,
                 (1.0f + sc.z) * (t[k].z * inv[k] * (1.0f + w.z)) + sh.z,
                 (1.0f + sc.w) * (t[k].w * inv[k] * (1.0f + w.w)) + sh.w);
    }
  };
#pragma unroll
  for (int u = 0; u < CACHE; ++u) {
    const int c = threadIdx.x + u * 256;
    if (c < H4) {
      float4 t[R];
#pragma unroll
      for (int k = 0; k < R; ++k) t[k] = v[k][u];
      emit(c, t);
    }
  }
  for (int c = threadIdx.x + CACHE * 256; c < H4; c += 256) {
    float4 t[R];
#pragma unroll
    for (int k = 0; k < R; ++k) t[k] = x[k][c];
    emit(c, t);
  }
}

// bf16 output, H a multiple of 8 up to 8 NT: each thread owns 8 consecutive columns of R rows (two
// 16-byte loads and one 16-byte store per row); NT threads cover the row. Every row's loads are issued
// before the first reduction and the rows' wave sums run side by side (issued row by row behind a
// branch, each row's loads had waited for the previous row's reduction).
template <int R, int NT>
__global__ void __launch_bounds__(NT) modnorm8_kernel(ModnormArgs p) {
  __shared__ float red[R][NT / 64];
  K2_LDS_CHECK(sizeof(red), 1);
  const int r0 = R * blockIdx.x;
  const int nr = min(R, p.rows - r0);
  const int c = threadIdx.x;  // 8-column chunk
  const bool on = c < (p.H >> 3);
  const int cc = on ? c : 0;  // a thread past the row loads chunk 0 and never stores
  const float4* x[R];
  bf16* y[R];
  int bb[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int r = k < nr ? r0 + k : r0;
    const int b = r / p.rows_per_b, i = r - b * p.rows_per_b;
    bb[k] = b;
    x[k] = (const float4*)(p.in + ((size_t)b * p.in_rows_per_b + p.in_row_off + i) * p.H);
    y[k] = (bf16*)p.out + (size_t)r * p.H;
  }
  float4 v[R][2];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    v[k][0] = x[k][2 * cc];
    v[k][1] = x[k][2 * cc + 1];
  }
  float ss[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (!on) v[k][0] = v[k][1] = make_float4(0.f, 0.f, 0.f, 0.f);
    ss[k] = v[k][0].x * v[k][0].x + v[k][0].y * v[k][0].y + v[k][0].z * v[k][0].z + v[k][0].w * v[k][0].w +
            v[k][1].x * v[k][1].x + v[k][1].y * v[k][1].y + v[k][1].z * v[k][1].z + v[k][1].w * v[k][1].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)  // the rows' wave sums side by side (wave_sum's order per row)
#pragma unroll
    for (int k = 0; k < R; ++k) ss[k] += __shfl_xor(ss[k], o);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < R; ++k) red[k][wv] = ss[k];
  }
  __syncthreads();
  if (!on) return;
  // (16-byte aligned vectors: checked by the host)
  auto ld8 = [](const float* q, float (&d)[8]) {
    const float4 a = reinterpret_cast<const float4*>(q)[0], b = reinterpret_cast<const float4*>(q)[1];
    d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w; d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
  };
  float w8[8] = {}, sc8[8] = {}, sh8[8] = {};
  if (p.w) ld8(p.w + 8 * c, w8);
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (k >= nr) break;
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < NT / 64; ++q) t += red[k][q];
    const float inv = rsqrtf(t / (float)p.H + p.eps);
    if (k == 0 || bb[k] != bb[k - 1]) {  // a new batch row: its modulation vectors
      if (p.scale) ld8(p.scale + (size_t)bb[k] * p.mod_stride + 8 * c, sc8);
      if (p.shift) ld8(p.shift + (size_t)bb[k] * p.mod_stride + 8 * c, sh8);
    }
    const float t8[8] = {v[k][0].x, v[k][0].y, v[k][0].z, v[k][0].w, v[k][1].x, v[k][1].y, v[k][1].z, v[k][1].w};
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((1.0f + sc8[e]) * (t8[e] * inv * (1.0f + w8[e])) + sh8[e]);
    *(bf16x8*)(y[k] + 8 * c) = o;
  }
}

constexpr int kModnormRows = 2;
// rows per workgroup of modnorm8_kernel, measured at 9216 x 6144 (same process, three runs each):
// 1 row 0.075 ms, 2 rows 0.067, 4 rows 0.065, 6 rows 0.074, 8 rows 0.077 (fewer waves per SIMD)
constexpr int kModnorm8Rows = 4;

template <int NT>
static hipError_t modnorm8(const ModnormArgs& p, hipStream_t s) {
  hipLaunchKernelGGL((modnorm8_kernel<kModnorm8Rows, NT>), dim3((p.rows + kModnorm8Rows - 1) / kModnorm8Rows), dim3(NT),
                     0, s, p);
  return hipGetLastError();
}

hipError_t modnorm(int dt, const ModnormArgs& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  const bool aligned = (((uintptr_t)p.w | (uintptr_t)p.scale | (uintptr_t)p.shift) & 15) == 0;
  if (dt == DT_BF16 && p.H % 8 == 0 && p.H <= 8 * 1024 && p.mod_stride % 4 == 0 && aligned) {
    const int h8 = p.H / 8;
    if (h8 <= 64) return modnorm8<64>(p, s);
    if (h8 <= 128) return modnorm8<128>(p, s);
    if (h8 <= 256) return modnorm8<256>(p, s);
    if (h8 <= 512) return modnorm8<512>(p, s);
    if (h8 <= 768) return modnorm8<768>(p, s);
    return modnorm8<1024>(p, s);
  }
  const int grid = (p.rows + kModnormRows - 1) / kModnormRows;
  if (dt == DT_BF16)
    hipLaunchKernelGGL((modnorm_kernel<bf16, kModnormRows>), dim3(grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((modnorm_kernel<float, kModnormRows>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

__global__ void modulation_kernel(const float* temb, int temb_stride, int chunk_stride, const float* table,
                                  float* mod, int B, int nchunks, int H) {
  const size_t n = (size_t)B * nchunks * H;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const int j = (int)(idx % H);
    const int c = (int)((idx / H) % nchunks);
    const int b = (int)(idx / ((size_t)H * nchunks));
    mod[idx] = temb[(size_t)b * temb_stride + (size_t)c * chunk_stride + j] + (table ? table[(size_t)c * H + j] : 0.0f);
  }
}

hipError_t modulation(const float* temb, int temb_stride, int chunk_stride, const float* table, float* mod, int B,
                      int nchunks, int H, hipStream_t s) {
  const size_t n = (size_t)B * nchunks * H;
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(modulation_kernel, dim3(blocks), dim3(256), 0, s, temb, temb_stride, chunk_stride, table, mod, B,
                     nchunks, H);
  return hipGetLastError();
}

__global__ void rope_table_kernel(const float* pos, int L, int a0, int a1, int a2, float theta, float* co, float* si) {
  const int half = (a0 + a1 + a2) / 2;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= L * half) return;
  const int l = idx / half, pi = idx - l * half;
  int a, i, d;
  if (pi < a0 / 2) { a = 0; i = pi; d = a0; }
  else if (pi < (a0 + a1) / 2) { a = 1; i = pi - a0 / 2; d = a1; }
  else { a = 2; i = pi - (a0 + a1) / 2; d = a2; }
  const double ang = (double)pos[(size_t)l * 3 + a] * pow((double)theta, -2.0 * i / d);
  co[idx] = (float)cos(ang);
  si[idx] = (float)sin(ang);
}

hipError_t rope_table(const float* pos, int L, int a0, int a1, int a2, float theta, float* cos_out, float* sin_out,
                      hipStream_t s) {
  const int n = L * ((a0 + a1 + a2) / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, pos, L, a0, a1, a2, theta, cos_out,
                     sin_out);
  return hipGetLastError();
}

template <typename T>
__global__ void time_embed_kernel(const float* t, int B, int dim, T* out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * dim) return;
  const int b = idx / dim, k = idx - b * dim, half = dim / 2;
  const int kk = k < half ? k : k - half;
  const double f = pow(10000.0, -(double)kk / half);
  const double arg = 1000.0 * (double)t[b] * f;
  out[idx] = to_t<T>((float)(k < half ? cos(arg) : sin(arg)));
}

hipError_t time_embed(int dt, const float* t, int B, int dim, void* out, hipStream_t s) {
  const int n = B * dim;
  if (n == 0) return hipSuccess;
  if (dt == DT_BF16)
    hipLaunchKernelGGL(time_embed_kernel<bf16>, dim3((n + 255) / 256), dim3(256), 0, s, t, B, dim, (bf16*)out);
  else
    hipLaunchKernelGGL(time_embed_kernel<float>, dim3((n + 255) / 256), dim3(256), 0, s, t, B, dim, (float*)out);
  return hipGetLastError();
}

__global__ void layer_compress_kernel(const float* x, const float* c, float* y, int rows, int nl, int D) {
  const size_t n = (size_t)rows * D;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const size_t r = idx / D;
    const int d = (int)(idx - r * D);
    const float* src = x + r * nl * D + d;
    float acc = 0.0f;
    for (int l = 0; l < nl; ++l) acc += c[l] * src[(size_t)l * D];
    y[idx] = acc;
  }
}

hipError_t layer_compress(const float* x, const float* c, float* y, int rows, int nl, int D, hipStream_t s) {
  const size_t n = (size_t)rows * D;
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL(layer_compress_kernel, dim3(blocks), dim3(256), 0, s, x, c, y, rows, nl, D);
  return hipGetLastError();
}

template <typename TI, typename TO>
__global__ void convert_kernel(const TI* in, TO* out, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    out[i] = to_t<TO>(to_f(in[i]));
}

template <typename TI, typename TO>
static hipError_t convert(const void* in, void* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL((convert_kernel<TI, TO>), dim3(blocks), dim3(256), 0, s, (const TI*)in, (TO*)out, n);
  return hipGetLastError();
}

hipError_t to_f32(int dt, const void* in, float* out, size_t n, hipStream_t s) {
  return dt == DT_BF16 ? convert<bf16, float>(in, out, n, s) : convert<float, float>(in, out, n, s);
}
hipError_t from_f32(int dt, const float* in, void* out, size_t n, hipStream_t s) {
  return dt == DT_BF16 ? convert<float, bf16>(in, out, n, s) : convert<float, float>(in, out, n, s);
}

// Guidance combine and Euler update of the sampler, fused: one pass over the latents, four floats
// per lane where the sizes allow.
__global__ void cfg_euler_kernel(const float* __restrict__ x, float* x_out, const float* __restrict__ vc,
                                 const float* __restrict__ vu, size_t n, float g, float dsigma) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 xv = reinterpret_cast<const float4*>(x)[i];
    const float4 c = reinterpret_cast<const float4*>(vc)[i];
    float4 v = c;
    if (vu) {
      const float4 u = reinterpret_cast<const float4*>(vu)[i];
      v = make_float4(c.x + g * (c.x - u.x), c.y + g * (c.y - u.y), c.z + g * (c.z - u.z), c.w + g * (c.w - u.w));
    }
    reinterpret_cast<float4*>(x_out)[i] =
        make_float4(xv.x + dsigma * v.x, xv.y + dsigma * v.y, xv.z + dsigma * v.z, xv.w + dsigma * v.w);
  }
  for (size_t i = 4 * n4 + (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float c = vc[i];
    const float v = vu ? c + g * (c - vu[i]) : c;
    x_out[i] = x[i] + dsigma * v;
  }
}

hipError_t cfg_euler(const float* x, float* x_out, const float* vc, const float* vu, size_t n, float g, float dsigma,
                     hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t work = (n + 3) / 4;
  const int blocks = (int)((work + 255) / 256 < 2048 ? (work + 255) / 256 : 2048);
  hipLaunchKernelGGL(cfg_euler_kernel, dim3(blocks), dim3(256), 0, s, x, x_out, vc, vu, n, g, dsigma);
  return hipGetLastError();
}

__global__ void fill_f32_kernel(float* out, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = v;
}

hipError_t fill_f32(float* out, int n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, out, n, v);
  return hipGetLastError();
}

// Block-causal reach: the end of each token's image-block run, by a suffix minimum over the run
// ends taken in chunks of 1024 positions from the back of the sequence (carry: the end of the run
// holding the first position of the chunk after the current one).
__global__ void __launch_bounds__(1024) block_reach_kernel(const int* __restrict__ ids, int L, int* __restrict__ reach) {
  __shared__ int sm[1024];
  K2_LDS_CHECK(sizeof(sm), 1);
  const int tid = threadIdx.x;
  int carry = INT_MAX;
  for (int c0 = ((L - 1) / 1024) * 1024; c0 >= 0; c0 -= 1024) {
    const int i = c0 + tid;
    int id = -1, v = INT_MAX;
    if (i < L) {
      id = ids[i];
      v = (i == L - 1 || ids[i + 1] != id) ? i : INT_MAX;  // i ends its run
    }
    sm[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // sm[t] = min(sm[t .. 1023])
      const int o = tid + off < 1024 ? sm[tid + off] : INT_MAX;
      __syncthreads();
      sm[tid] = min(sm[tid], o);
      __syncthreads();
    }
    if (i < L) reach[i] = id >= 0 ? min(sm[tid], carry) : i;
    const int first = min(sm[0], carry);
    __syncthreads();
    carry = first;
  }
}

hipError_t block_reach(const int* ids, int L, int* reach, hipStream_t s) {
  if (L <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_reach_kernel, dim3(1), dim3(1024), 0, s, ids, L, reach);
  return hipGetLastError();
}

}  // namespace k2
