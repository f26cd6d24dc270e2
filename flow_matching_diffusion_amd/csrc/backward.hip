// Backward pass of the single-stream block (gfx950): the kernels that are not GEMMs.
//
// The block's gradient follows the chain rule through the forward's steps in reverse, the forward
// recomputed from the block input (architecture article, data flow of §四; its §六 test matrix
// trains the model with gradient checkpointing). Every matrix product of the backward runs on the
// forward's GEMM kernel with a plain epilogue; these kernels supply what the products need:
//
//   transpose      — batched 2D transposes (weights and activations into the K-contiguous layout
//                    the GEMM reads; q, dO and k per head for the attention backward)
//   gated_add      — h1 = h + gate_b * y (the residual after attention, from the recomputed y)
//   gated_grad     — d(branch) = gate_b * dh in the operand dtype, and per-chunk column sums of
//                    dh * branch (the gate's gradient)
//   swiglu_bwd     — dgate = da * up * silu'(gate), dup = da * silu(gate)
//   norm_bwd       — RMSNorm + modulation backward over whole rows, plus per-chunk column sums
//                    for the norm weight and the scale / shift gradients
//   gate_bwd       — sigmoid output gate backward and Delta = rowsum(dO * O) per (row, head)
//   attn_bwd_dq    — dQ = dS K / sqrt(hd), one wave per 32 queries of one head
//   attn_bwd_dkv   — dK = dS^T Q / sqrt(hd) and dV = P^T dO over the query heads of a kv head,
//                    one wave per 32 keys
//   qknorm_bwd     — the RoPE rotation's transpose, then the per-head RMSNorm backward
//   reduce_rows    — sums of the per-chunk partials
//
// Attention backward, with P = softmax(S), S = Q K^T / sqrt(hd) under the key mask, O = P V:
// dV = P^T dO, dP = dO V^T, dS = P (dP - Delta), Delta = rowsum(dO * O); P is recomputed from the
// forward's per-row log-sum-exp. Both kernels use the 16x16 matrix-core block of k2_device.h for
// bf16 and float32 operands, with the tiles a workgroup's waves share staged in LDS.
#include <algorithm>

#include "k2_device.h"
#include "k2_kernels.h"

namespace k2 {

namespace {

template <typename T>
__device__ __forceinline__ typename FragOf<T>::type ld_frag(const T* p) {
  typename FragOf<T>::type f;
  if constexpr (sizeof(T) == 2) {
    f = *(const bf16x8*)p;
  } else {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  return f;
}

// the first n (0 <= n <= 8) elements of p, zeros after (elements at or past n are not read)
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type ld_frag_n(const T* p, int n) {
  typename FragOf<T>::type f;
  if (n >= 8) return ld_frag<T>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = e < n ? p[e] : (T)0.0f;
  return f;
}

template <typename T>
__device__ __forceinline__ typename FragOf<T>::type zero_frag() {
  typename FragOf<T>::type f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (T)0.0f;
  return f;
}

// row index of 16-row block kb, accumulator row rho -> position in a 32-wide tile
__device__ __forceinline__ int perm32(int kb, int rho) { return 8 * (rho >> 2) + 4 * kb + (rho & 3); }

// Position of chunk cc of row r in an LDS tile of 16-chunk rows (bf16, head_dim 128). A fragment read
// takes the 16 rows perm32(kb, 0..15) = {0-3, 8-11, 16-19, 24-27} (+4 for kb = 1) at one chunk: an
// XOR of the chunk with row bits 0-1 and 3-4 puts those rows in 16 different 16-byte bank groups.
// Rows padded by one chunk instead (the other tiles' layout) put rows r and r + 8 in the same banks:
// the counters read hundreds of millions of conflict cycles per launch that way.
template <bool SWZ>
__device__ __forceinline__ int tile_chunk(int r, int cc) {
  return SWZ ? cc ^ ((r & 3) | (((r >> 3) & 3) << 2)) : cc;
}

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int N>
__device__ __forceinline__ float group_sum(float v) {  // over N consecutive lanes (N <= 64)
#pragma unroll
  for (int o = 1; o < N; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Batched transpose: for z < Z, dst_z[c][r] = src_z[r][c] (r < R, c < C) and dst_z[c][r] = 0 for
// R <= r < Rpad. src_z = src + (z / zdiv) * sz0 + (z % zdiv) * sz1, dst_z likewise.
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) transpose_kernel(TransposeArgs p) {
  __shared__ T tile[64][65];
  K2_LDS_CHECK(sizeof(tile), 1);
  const int z = blockIdx.z;
  const T* src = (const T*)p.src + (size_t)(z / p.zdiv) * p.sz0 + (size_t)(z % p.zdiv) * p.sz1;
  T* dst = (T*)p.dst + (size_t)(z / p.zdiv) * p.dz0 + (size_t)(z % p.zdiv) * p.dz1;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + ty + 4 * i, c = c0 + tx;
    tile[ty + 4 * i][tx] = (r < p.R && c < p.C) ? src[(size_t)r * p.lds + c] : (T)0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = c0 + ty + 4 * i, r = r0 + tx;
    if (c < p.C && r < p.Rpad) dst[(size_t)c * p.ldd + r] = tile[tx][ty + 4 * i];
  }
}

// The same transpose in 16-byte chunks of EPC elements, for operands whose row strides, batch
// offsets, C and Rpad are multiples of EPC and whose base pointers are 16-byte aligned. A lane
// loads one chunk of a source row (8 lanes cover a 128-byte row segment) and stores one chunk of a
// destination row, gathered from EPC consecutive source rows of the LDS tile. Chunk cc of tile row
// r sits at cc ^ ((r / EPC) % CPR): the chunk writes fill whole rows, and the gathers of a lane
// group (EPC rows apart, one column) fall in distinct banks. The element-wise kernel above moved 2
// or 4 bytes per lane per memory instruction and ran at about 2.5 TB/s.
template <typename T>
__global__ void __launch_bounds__(256) transpose_vec_kernel(TransposeArgs p) {
  constexpr int EPC = 16 / sizeof(T);  // elements per chunk
  constexpr int CPR = 64 / EPC;        // chunks per 64-element tile row
  __shared__ uint4 tile[64 * CPR];
  K2_LDS_CHECK(sizeof(tile), 1);
  const int z = blockIdx.z;
  const T* src = (const T*)p.src + (size_t)(z / p.zdiv) * p.sz0 + (size_t)(z % p.zdiv) * p.sz1;
  T* dst = (T*)p.dst + (size_t)(z / p.zdiv) * p.dz0 + (size_t)(z % p.zdiv) * p.dz1;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int k = 0; k < 64 * CPR / 256; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int row = u / CPR, cc = u % CPR;
    const int r = r0 + row, c = c0 + cc * EPC;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < p.R && c < p.C) v = *(const uint4*)(src + (size_t)r * p.lds + c);
    tile[row * CPR + (cc ^ ((row / EPC) % CPR))] = v;
  }
  __syncthreads();
  const T* t = reinterpret_cast<const T*>(tile);
#pragma unroll
  for (int k = 0; k < 64 * CPR / 256; ++k) {
    const int u = threadIdx.x + 256 * k;
    const int col = u / CPR, rc = u % CPR;  // destination row c0 + col, source rows r0 + EPC rc ..
    const int c = c0 + col, r = r0 + rc * EPC;
    if (c < p.C && r < p.Rpad) {
      union { uint4 v; T e[EPC]; } out;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int row = rc * EPC + e;  // (row / EPC) % CPR == rc
        out.e[e] = t[(row * CPR + ((col / EPC) ^ rc)) * EPC + col % EPC];
      }
      *(uint4*)(dst + (size_t)c * p.ldd + r) = out.v;
    }
  }
}

template <typename T>
static bool transpose_vec_ok(const TransposeArgs& p) {
  constexpr size_t EPC = 16 / sizeof(T);
  const bool aligned = ((uintptr_t)p.src % 16 == 0) && ((uintptr_t)p.dst % 16 == 0);
  return aligned && p.C % EPC == 0 && p.Rpad % EPC == 0 && p.lds % EPC == 0 && p.ldd % EPC == 0 &&
         p.sz0 % EPC == 0 && p.sz1 % EPC == 0 && p.dz0 % EPC == 0 && p.dz1 % EPC == 0;
}

hipError_t transpose(int dt, const TransposeArgs& p, hipStream_t s) {
  if (p.R <= 0 || p.C <= 0 || p.Z <= 0) return hipSuccess;
  if (p.Rpad < p.R || p.ldd < p.Rpad || p.zdiv <= 0) return hipErrorInvalidValue;
  dim3 grid((p.C + 63) / 64, (p.Rpad + 63) / 64, p.Z);
  if (dt == DT_BF16) {
    if (transpose_vec_ok<bf16>(p))
      hipLaunchKernelGGL(transpose_vec_kernel<bf16>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, p);
  } else {
    if (transpose_vec_ok<float>(p))
      hipLaunchKernelGGL(transpose_vec_kernel<float>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// h1 = h + gate[b] * y over (M, H) float32, b = row / L (gate NULL: 1)
// ---------------------------------------------------------------------------------------------
__global__ void gated_add_kernel(const float* __restrict__ h, const float* __restrict__ y, const float* gate,
                                 int gate_stride, int L, int M, int H, float* __restrict__ out) {
  const size_t n4 = (size_t)M * H / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const size_t e = 4 * i;
    const int row = (int)(e / H), col = (int)(e - (size_t)row * H);
    const float4 a = *(const float4*)(h + e), v = *(const float4*)(y + e);
    float4 g = make_float4(1.f, 1.f, 1.f, 1.f);
    if (gate) g = *(const float4*)(gate + (size_t)(row / L) * gate_stride + col);
    *(float4*)(out + e) = make_float4(a.x + g.x * v.x, a.y + g.y * v.y, a.z + g.z * v.z, a.w + g.w * v.w);
  }
}

hipError_t gated_add(const float* h, const float* y, const float* gate, int gate_stride, int L, int M, int H,
                     float* out, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const size_t n4 = (size_t)M * H / 4;
  const int blocks = (int)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  hipLaunchKernelGGL(gated_add_kernel, dim3(blocks), dim3(256), 0, s, h, y, gate, gate_stride, L, M, H, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Gated branch gradient: out[m] = T(gate_b * dh[m]) and part[chunk][col] = sum over the chunk's rows
// of dh * br (chunks: rows [b L + c RC, ...) within one batch row; chunk index b * ncb + c).
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(256) gated_grad_kernel(GatedGradArgs p) {
  const int c4 = blockIdx.x * 256 + threadIdx.x;  // float4 column
  const int chunk = blockIdx.y;
  const int b = chunk / p.ncb, c = chunk - b * p.ncb;
  const int l0 = c * p.RC, l1 = min(p.L, l0 + p.RC);
  if (4 * c4 >= p.H) return;
  float4 g = make_float4(1.f, 1.f, 1.f, 1.f);
  if (p.gate) g = *(const float4*)(p.gate + (size_t)b * p.gate_stride + 4 * c4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int l = l0; l < l1; ++l) {
    const size_t e = ((size_t)b * p.L + l) * p.H + 4 * c4;
    const float4 d = *(const float4*)(p.dh + e);
    if (p.br) {
      const float4 v = *(const float4*)(p.br + e);
      acc.x += d.x * v.x; acc.y += d.y * v.y; acc.z += d.z * v.z; acc.w += d.w * v.w;
    }
    T* o = (T*)p.out + e;
    o[0] = (T)(g.x * d.x); o[1] = (T)(g.y * d.y); o[2] = (T)(g.z * d.z); o[3] = (T)(g.w * d.w);
  }
  if (p.part) *(float4*)(p.part + (size_t)chunk * p.H + 4 * c4) = acc;
}

hipError_t gated_grad(int dt, const GatedGradArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.L <= 0) return hipSuccess;
  if (p.H % 4 || p.RC <= 0 || p.ncb != (p.L + p.RC - 1) / p.RC) return hipErrorInvalidValue;
  dim3 grid((p.H / 4 + 255) / 256, p.B * p.ncb);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(gated_grad_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(gated_grad_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// 8 consecutive elements (16-byte aligned for bf16, 32-byte for float) to / from float
__device__ __forceinline__ void load8f(const bf16* p, float (&v)[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ __forceinline__ void load8f(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8*>(p) = x;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------------------------
// SwiGLU backward: dgu[m][i] = T(da * up * silu'(g)), dgu[m][I + i] = T(da * silu(g)),
// silu'(x) = s(x) (1 + x (1 - s(x))). da, g, up: (M, I) float32; dgu: (M, 2I).
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ void swiglu_bwd_kernel(const float* __restrict__ da, const float* __restrict__ gt,
                                  const float* __restrict__ up, int M, int I, T* __restrict__ dgu) {
  const size_t n = (size_t)M * I;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const size_t m = e / I, i = e - m * I;
    const float x = gt[e], u = up[e], d = da[e];
    const float sg = sigm(x);
    dgu[m * 2 * I + i] = (T)(d * u * sg * (1.0f + x * (1.0f - sg)));
    dgu[m * 2 * I + I + i] = (T)(d * x * sg);
  }
}

// The same, 8 consecutive elements per thread with 16- and 32-byte accesses (I a multiple of 8).
template <typename T>
__global__ void swiglu_bwd8_kernel(const float* __restrict__ da, const float* __restrict__ gt,
                                   const float* __restrict__ up, int M, int I, T* __restrict__ dgu) {
  const size_t n8 = (size_t)M * I / 8;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < n8; c += (size_t)gridDim.x * blockDim.x) {
    const size_t e = 8 * c, m = e / I, i = e - m * I;
    float x[8], u[8], d[8], dg[8], du[8];
    load8f(gt + e, x);
    load8f(up + e, u);
    load8f(da + e, d);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sg = sigm(x[k]);
      dg[k] = d[k] * u[k] * sg * (1.0f + x[k] * (1.0f - sg));
      du[k] = d[k] * x[k] * sg;
    }
    store8(dgu + m * 2 * I + i, dg);
    store8(dgu + m * 2 * I + I + i, du);
  }
}

hipError_t swiglu_bwd(int dt, const float* da, const float* gt, const float* up, int M, int I, void* dgu,
                      hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const size_t n = (size_t)M * I;
  if (I % 8 == 0) {
    const int blocks = (int)((n / 8 + 255) / 256 < 8192 ? (n / 8 + 255) / 256 : 8192);
    if (dt == DT_BF16)
      hipLaunchKernelGGL(swiglu_bwd8_kernel<bf16>, dim3(blocks), dim3(256), 0, s, da, gt, up, M, I, (bf16*)dgu);
    else
      hipLaunchKernelGGL(swiglu_bwd8_kernel<float>, dim3(blocks), dim3(256), 0, s, da, gt, up, M, I, (float*)dgu);
    return hipGetLastError();
  }
  const int blocks = (int)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16>, dim3(blocks), dim3(256), 0, s, da, gt, up, M, I, (bf16*)dgu);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, da, gt, up, M, I, (float*)dgu);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// RMSNorm + modulation backward. Forward: n = x r (1 + w), r = 1/sqrt(mean(x^2) + eps),
// out = (1 + sc_b) n + sh_b. For the gradient dout of out: dn = (1 + sc_b) dout, g = dn (1 + w),
// dx = r g - x r^3 sum(g x) / H, added to dres into dx_out. Partials per chunk of rows (one
// batch row each): pw = sum dn x r, psc = sum dout n, psh = sum dout. One workgroup per chunk,
// each row held in registers (H <= 8192).
// ---------------------------------------------------------------------------------------------
// NT threads per workgroup and CACHE float4s of each row per thread (H <= 4 NT CACHE): 1024 x 2
// for the 6144-wide rows of the block, 108 registers, 16 waves per compute unit. The residual
// gradient is loaded with x and dout, so a row's three reads are in flight together; the two row
// sums go through LDS slots that alternate between rows, one barrier per row.
template <int NT, int CACHE>
__global__ void __launch_bounds__(NT) norm_bwd_kernel(NormBwdArgs p) {
  constexpr int NW = NT / 64;  // waves
  __shared__ float red[2][2][NW];
  K2_LDS_CHECK(sizeof(red), 1);
  const int chunk = blockIdx.x;
  const int b = chunk / p.ncb, c = chunk - b * p.ncb;
  const int l0 = c * p.RC, l1 = min(p.L, l0 + p.RC);
  const int H4 = p.H >> 2, tid = threadIdx.x, wv = tid >> 6;
  const float4* w4 = (const float4*)p.w;
  const float4* sc4 = p.scale ? (const float4*)(p.scale + (size_t)b * p.mod_stride) : nullptr;
  float4 pw[CACHE], psc[CACHE], psh[CACHE], mw[CACHE], ms[CACHE];
#pragma unroll
  for (int u = 0; u < CACHE; ++u) {
    pw[u] = psc[u] = psh[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int cc = tid + u * NT;
    mw[u] = ms[u] = make_float4(1.f, 1.f, 1.f, 1.f);
    if (cc < H4) {
      if (w4) { const float4 t = w4[cc]; mw[u] = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w); }
      if (sc4) { const float4 t = sc4[cc]; ms[u] = make_float4(1.f + t.x, 1.f + t.y, 1.f + t.z, 1.f + t.w); }
    }
  }
  for (int l = l0; l < l1; ++l) {
    const size_t row = (size_t)b * p.L + l;
    const float4* x4 = (const float4*)(p.x + row * p.H);
    const float4* d4 = (const float4*)(p.dout + row * p.H);
    const float4* res4 = p.dres ? (const float4*)(p.dres + row * p.H) : nullptr;
    float4 xv[CACHE], dv[CACHE], rv[CACHE];
#pragma unroll
    for (int u = 0; u < CACHE; ++u) {
      const int cc = tid + u * NT;
      xv[u] = dv[u] = rv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cc < H4) {
        xv[u] = x4[cc];
        dv[u] = d4[cc];
        if (res4) rv[u] = res4[cc];
      }
    }
    float ss = 0.0f, dot = 0.0f;
#pragma unroll
    for (int u = 0; u < CACHE; ++u) {
      ss += xv[u].x * xv[u].x + xv[u].y * xv[u].y + xv[u].z * xv[u].z + xv[u].w * xv[u].w;
      // g = dout (1 + sc) (1 + w)
      dot += dv[u].x * ms[u].x * mw[u].x * xv[u].x + dv[u].y * ms[u].y * mw[u].y * xv[u].y +
             dv[u].z * ms[u].z * mw[u].z * xv[u].z + dv[u].w * ms[u].w * mw[u].w * xv[u].w;
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const int slot = (l - l0) & 1;  // a row's slots are rewritten two rows later, after a barrier
    if ((tid & 63) == 0) {
      red[slot][0][wv] = ss;
      red[slot][1][wv] = dot;
    }
    __syncthreads();
    ss = 0.0f;
    dot = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      ss += red[slot][0][k];
      dot += red[slot][1][k];
    }
    const float r = rsqrtf(ss / (float)p.H + p.eps);
    const float k3 = r * r * r * dot / (float)p.H;
    float4* o4 = (float4*)(p.dx + row * p.H);
#pragma unroll
    for (int u = 0; u < CACHE; ++u) {
      const int cc = tid + u * NT;
      if (cc >= H4) continue;
      const float4 x = xv[u], d = dv[u], m1 = ms[u], m2 = mw[u];
      float4 res = rv[u];
      res.x += r * d.x * m1.x * m2.x - x.x * k3;
      res.y += r * d.y * m1.y * m2.y - x.y * k3;
      res.z += r * d.z * m1.z * m2.z - x.z * k3;
      res.w += r * d.w * m1.w * m2.w - x.w * k3;
      o4[cc] = res;
      pw[u].x += d.x * m1.x * x.x * r; pw[u].y += d.y * m1.y * x.y * r;
      pw[u].z += d.z * m1.z * x.z * r; pw[u].w += d.w * m1.w * x.w * r;
      psc[u].x += d.x * x.x * r * m2.x; psc[u].y += d.y * x.y * r * m2.y;
      psc[u].z += d.z * x.z * r * m2.z; psc[u].w += d.w * x.w * r * m2.w;
      psh[u].x += d.x; psh[u].y += d.y; psh[u].z += d.z; psh[u].w += d.w;
    }
  }
#pragma unroll
  for (int u = 0; u < CACHE; ++u) {
    const int cc = tid + u * NT;
    if (cc >= H4) continue;
    if (p.pw) ((float4*)(p.pw + (size_t)chunk * p.H))[cc] = pw[u];
    if (p.psc) ((float4*)(p.psc + (size_t)chunk * p.H))[cc] = psc[u];
    if (p.psh) ((float4*)(p.psh + (size_t)chunk * p.H))[cc] = psh[u];
  }
}

hipError_t norm_bwd(const NormBwdArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.L <= 0) return hipSuccess;
  if (p.H % 4 || p.H > 4 * 1024 * 2 || p.RC <= 0 || p.ncb != (p.L + p.RC - 1) / p.RC) return hipErrorInvalidValue;
  const int H4 = p.H / 4;
  const dim3 grid(p.B * p.ncb);
  if (H4 <= 512)
    hipLaunchKernelGGL((norm_bwd_kernel<512, 1>), grid, dim3(512), 0, s, p);
  else if (H4 <= 1024)
    hipLaunchKernelGGL((norm_bwd_kernel<512, 2>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((norm_bwd_kernel<1024, 2>), grid, dim3(1024), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Output gate backward and Delta, per (row, head): do = T(dog * s(g)), dg = T(dog * o * s (1 - s)),
// delta[(b nh + h) L + l] = sum_d do * o. HD/8 threads per (row, head), 8 head dims each.
// ---------------------------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(256) gate_bwd_kernel(GateBwdArgs p) {
  constexpr int TPI = HD / 8;  // threads per item
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const long item = tid / TPI;
  const int ch = tid % TPI;
  const long nitems = (long)p.M * p.nh;
  if (item >= nitems) return;  // TPI divides 64: whole groups leave together
  const int m = (int)(item / p.nh), h = (int)(item - (long)m * p.nh);
  const int col = h * HD + 8 * ch;
  const float* dog = p.dog + (size_t)m * p.nq + col;
  const T* g = (const T*)p.g + (size_t)m * p.nq + col;
  const T* o = (const T*)p.o + (size_t)m * p.nq + col;
  T* dout = (T*)p.dout + (size_t)m * p.nq + col;
  T* dg = (T*)p.dg + (size_t)m * p.ldg + col;
  // 16-byte loads and stores (written as element loops between stores, they stayed 2-byte accesses)
  float gv[8], ov[8], dv[8], dov[8], dgv[8];
  load8f(g, gv);
  load8f(o, ov);
  load8f(dog, dv);
  float dsum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float s = sigm(gv[e]);
    dov[e] = (float)(T)(dv[e] * s);  // dO as the operand dtype holds it
    dgv[e] = dv[e] * ov[e] * s * (1.0f - s);
    dsum += dov[e] * ov[e];
  }
  store8(dout, dov);
  store8(dg, dgv);
  dsum = group_sum<TPI>(dsum);
  if (ch == 0) {
    const int b = m / p.L, l = m - b * p.L;
    p.delta[((size_t)b * p.nh + h) * p.L + l] = dsum;
  }
}

hipError_t gate_bwd(int dt, const GateBwdArgs& p, hipStream_t s) {
  if (p.M <= 0) return hipSuccess;
  const long threads = (long)p.M * p.nh * (p.hd / 8);
  const int blocks = (int)((threads + 255) / 256);
  if (p.hd == 128 && dt == DT_BF16)
    hipLaunchKernelGGL((gate_bwd_kernel<bf16, 128>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 128)
    hipLaunchKernelGGL((gate_bwd_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 64 && dt == DT_BF16)
    hipLaunchKernelGGL((gate_bwd_kernel<bf16, 64>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 64)
    hipLaunchKernelGGL((gate_bwd_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Attention backward. Two kernels, both on 16x16 matrix-core blocks (bf16 or float32 operands),
// with the tiles all four waves of a workgroup use staged once in LDS (two stages, one barrier per
// tile; rows padded by one 16-byte chunk so that 16 rows read at one chunk hit different banks).
// The permuted row order perm32 (accumulator row 4g + r of 16-row block kb is index 8g + 4kb + r
// of the 32-wide tile) hands every lane group 8 consecutive keys or queries, which are the k slots
// of the next product's register operand.
//
// dQ: a workgroup is (batch row, kv head, 32 * 4/G queries); wave w takes query head
// kvh G + w % G and 32 queries (two 16-query column blocks). Per 32-key tile:
//   S^T = K Q^T      A: K rows from LDS,   B: Q^T (registers, loaded once)
//   dP^T = V dO^T    A: V rows from LDS,   B: dO^T (registers)
//   P^T = exp2(S^T scale_log2 - lse2[q]) on allowed keys, dS^T = P^T (dP^T - Delta[q])
//   dQ^T += K^T dS^T A: K^T rows from LDS, B: dS^T from registers
// dK, dV: a workgroup is (batch row, kv head, 128 keys); wave w takes 32 keys (two 16-key column
// blocks) and runs over the G query heads of the kv head and every 32-query tile:
//   S = Q K^T        A: Q rows from LDS,   B: K^T (registers)
//   dP = dO V^T      A: dO rows from LDS,  B: V^T (registers)
//   P, dS as above (lse and Delta of the tile's queries staged in LDS)
//   dV^T += dO^T P   A: dO^T rows from LDS, B: P from registers
//   dK^T += Q^T dS   A: Q^T rows from LDS,  B: dS from registers
// ---------------------------------------------------------------------------------------------
namespace {

// zero the elements at positions >= n of a 16-byte chunk of T (0 <= n)
template <typename T>
__device__ __forceinline__ uint4 chunk_keep(uint4 v, int n) {
  constexpr int E = 16 / sizeof(T);
  T* e = reinterpret_cast<T*>(&v);
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (i >= n) e[i] = (T)0.0f;
  return v;
}

// 16 bytes at p, or zeros when !ok (p is then not read)
__device__ __forceinline__ uint4 ld16_or_zero(const void* p, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) v = *(const uint4*)p;
  return v;
}

// the 8-element fragment starting at chunk `chunk` of an LDS row
template <typename T>
__device__ __forceinline__ typename FragOf<T>::type lds_frag(const uint4* row, int chunk) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, row[chunk]);
  } else {
    const uint4 a = row[chunk], b = row[chunk + 1];
    f32x8 f;
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
    return f;
  }
}

}  // namespace

constexpr int kBwdTextTiles = 512;  // 32-key text tiles the dQ pass's validity bits hold: T <= 16384

template <typename T, int HD, int G>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(AttnBwdArgs p, float scale_log2, float scale) {
  typedef typename FragOf<T>::type Frag;
  constexpr int E = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int NC = HD / 32;            // k steps over head_dim
  constexpr int NDB = HD / 16;           // 16-row head-dim blocks of dQ^T
  constexpr int RCH = HD / E;                // chunks per K / V row
  constexpr bool SWZ = sizeof(T) == 2 && RCH == 16;  // bf16 head_dim 128: swizzled rows (tile_chunk)
  constexpr int RP = SWZ ? RCH : RCH + 1;    // row pitch
  constexpr int TCH = 32 / E, TP = TCH + 1;  // chunks per K^T row (32 keys), row pitch
  constexpr int NKV = 32 * RCH / 256, NT = HD * TCH / 256;  // chunks per thread per tile
  constexpr int QW = 32 * (4 / G);       // queries per workgroup
  static_assert(NKV >= 1 && NT >= 1, "tile / thread mismatch");
  __shared__ uint4 sK[2][32 * RP], sV[2][32 * RP], sT[2][HD * TP];
  __shared__ uint32_t sMb[kBwdTextTiles];  // bit j of word t: text key 32t + j may be attended
  // at most one workgroup's LDS per compute unit; two per compute unit (the launch bounds' aim) in bf16
  K2_LDS_CHECK(sizeof(sK) + sizeof(sV) + sizeof(sT) + sizeof(sMb), sizeof(T) == 2 ? 2 : 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int head = kvh * G + wave % G;
  const int q0 = blockIdx.x * QW + (wave / G) * 32;
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const bool active = q0 < L;  // wave-uniform; an idle wave still loads its share and meets the barriers

  Frag qf[2][NC], df[2][NC];
  float lse[2], dl[2];
#pragma unroll
  for (int qc = 0; qc < 2; ++qc) {
    const int qi = q0 + 16 * qc + c;
    const bool ok = qi < L;
    const size_t row = (size_t)(b * L + (ok ? qi : 0)) * ldq + head * HD + 8 * g;
#pragma unroll
    for (int kc = 0; kc < NC; ++kc) {
      qf[qc][kc] = ok ? ld_frag<T>((const T*)p.q + row + 32 * kc) : zero_frag<T>();
      df[qc][kc] = ok ? ld_frag<T>((const T*)p.dout + row + 32 * kc) : zero_frag<T>();
    }
    const size_t rs = ((size_t)b * p.nh + head) * L + (ok ? qi : 0);
    lse[qc] = ok ? p.lse[rs] : INFINITY;
    dl[qc] = ok ? p.delta[rs] : 0.0f;
  }
  // validity bits of the text tiles, once per workgroup (one wave ballot covers two tiles); the key
  // loop reads its tile's word instead of loading mask bytes per tile
  const int ntt = (T_ + 31) / 32;
  for (int u = wave; 2 * u < ntt; u += 4) {
    const int key = 64 * u + lane;
    const bool ok = key < L && (key >= T_ || !p.mask || p.mask[(size_t)b * T_ + key] != 0);
    const uint64_t bits = __ballot(ok);
    if (lane == 0) {
      sMb[2 * u] = (uint32_t)bits;
      if (2 * u + 1 < ntt) sMb[2 * u + 1] = (uint32_t)(bits >> 32);
    }
  }
  f32x4 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* kg = (const T*)p.k + (size_t)b * L * ldk + kvh * HD;
  const T* vg = (const T*)p.v + (size_t)b * L * ldk + kvh * HD;
  const T* tg = (const T*)p.kt + (size_t)(b * p.nkv + kvh) * HD * p.ldt;
  // one register set: tile loads run one tile ahead of the products, which keeps the kernel within
  // 256 registers, so two waves share a SIMD and one's exponentials overlap the other's matrix-core
  // work (two sets, two tiles ahead, took 324 registers and one wave per SIMD: 2.9 ms at block1024)
  uint4 rk[1][NKV], rv[1][NKV], rt[1][NT];
  int rt0[1] = {0};  // first key of the loaded tile
  // Tile loads are branch-free (buffer resources: keys past L read zero) and the K^T chunk at the
  // sequence end is trimmed at the LDS store, where the tile's loads are waited for anyway. Key
  // validity comes from the bits above. A mask byte loaded per tile in a branch and tested at once
  // made wave 0 wait for it right after issuing the tile's loads, and the workgroup with it at the
  // next barrier.
  const rsrc_t krs = make_rsrc(kg, ((size_t)(L - 1) * ldk + HD) * sizeof(T));
  const rsrc_t vrs = make_rsrc(vg, ((size_t)(L - 1) * ldk + HD) * sizeof(T));
  const rsrc_t trs = make_rsrc(tg, (size_t)HD * p.ldt * sizeof(T));
#define K2_DQ_GLOAD(RS, t)                                                                         \
  do {                                                                                             \
    const int t0_ = 32 * (t);                                                                      \
    rt0[RS] = t0_;                                                                                 \
    _Pragma("unroll") for (int i = 0; i < NKV; ++i) {                                              \
      const int ch_ = tid + 256 * i, row_ = ch_ / RCH, cc_ = ch_ % RCH, key_ = t0_ + row_;          \
      const uint32_t off_ = key_ < L ? (uint32_t)(key_ * ldk + cc_ * E) * (uint32_t)sizeof(T) : kOOB; \
      rk[RS][i] = bload(krs, off_);                                                                \
      rv[RS][i] = bload(vrs, off_);                                                                \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                               \
      const int ch_ = tid + 256 * i, d_ = ch_ / TCH, cc_ = ch_ % TCH, k0_ = t0_ + cc_ * E;          \
      rt[RS][i] = bload(trs, k0_ < L ? (uint32_t)(d_ * p.ldt + k0_) * (uint32_t)sizeof(T) : kOOB); \
    }                                                                                              \
  } while (0)
#define K2_DQ_LSTORE(RS, ST)                                                                       \
  do {                                                                                             \
    _Pragma("unroll") for (int i = 0; i < NKV; ++i) {                                              \
      const int ch_ = tid + 256 * i, row_ = ch_ / RCH, cc_ = ch_ % RCH;                             \
      sK[ST][row_ * RP + tile_chunk<SWZ>(row_, cc_)] = rk[RS][i];                                  \
      sV[ST][row_ * RP + tile_chunk<SWZ>(row_, cc_)] = rv[RS][i];                                  \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                               \
      const int ch_ = tid + 256 * i, d_ = ch_ / TCH, cc_ = ch_ % TCH, k0_ = rt0[RS] + cc_ * E;      \
      /* the workspace past L holds anything */                                                    \
      sT[ST][d_ * TP + cc_] = k0_ < L && k0_ + E > L ? chunk_keep<T>(rt[RS][i], L - k0_) : rt[RS][i]; \
    }                                                                                              \
  } while (0)

  const int nt = (L + 31) / 32;
  K2_DQ_GLOAD(0, 0);
  K2_DQ_LSTORE(0, 0);
  __syncthreads();
  // Tile t: its loads for tile t + 1 are issued first, then the products from LDS stage t & 1, then
  // tile t + 1 goes to stage (t + 1) & 1 (read by tile t - 1 before the last barrier). The loop runs
  // two tiles per turn so that the stages are fixed at compile time.
  // One tile: S = Q K^T; dP = dO V^T with P = exp2(S log2(e)/sqrt(hd) - lse + key bias) computed
  // alongside (the matrix cores have independent work during the exponentials); dS = P (dP - Delta);
  // dQ += dS K.
  auto tile = [&](int t, int st) {
    if (active) {
      // keys 8g + 4kb + r of the tile: bias 0 if the key may be attended, -inf if not
      const int t0 = 32 * t;
      const uint32_t vb = t < ntt ? sMb[t] : (t0 + 32 <= L ? ~0u : (1u << (L - t0)) - 1u);
      float4 kbias[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t nib = vb >> (8 * g + 4 * kb);
        kbias[kb] = make_float4((nib & 1u) ? 0.0f : -INFINITY, (nib & 2u) ? 0.0f : -INFINITY,
                                (nib & 4u) ? 0.0f : -INFINITY, (nib & 8u) ? 0.0f : -INFINITY);
      }
      f32x4 s[2][2], dp[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kro = perm32(kb, c);
        const uint4* kr = sK[st] + kro * RP;
#pragma unroll
        for (int kc = 0; kc < NC; ++kc) {
          const Frag ka = lds_frag<T>(kr, tile_chunk<SWZ>(kro, (32 * kc + 8 * g) / E));
#pragma unroll
          for (int qc = 0; qc < 2; ++qc) s[kb][qc] = mma16(s[kb][qc], ka, qf[qc][kc]);
        }
      }
      float pv[2][8];  // P for query block qc: entry 4 kb + r
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dp[kb][0] = dp[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int vro = perm32(kb, c);
        const uint4* vr = sV[st] + vro * RP;
        const float bias[4] = {kbias[kb].x, kbias[kb].y, kbias[kb].z, kbias[kb].w};
#pragma unroll
        for (int kc = 0; kc < NC; ++kc) {
          const Frag va = lds_frag<T>(vr, tile_chunk<SWZ>(vro, (32 * kc + 8 * g) / E));
#pragma unroll
          for (int qc = 0; qc < 2; ++qc) dp[kb][qc] = mma16(dp[kb][qc], va, df[qc][kc]);
          // 8 / NC exponentials of key block kb per step
#pragma unroll
          for (int x = kc * 8 / NC; x < (kc + 1) * 8 / NC; ++x) {
            const int qc = x >> 2, r = x & 3;
            pv[qc][4 * kb + r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qc][r], scale_log2, -lse[qc]) + bias[r]);
          }
        }
      }
      Frag dsf[2];
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = pv[qc][e] * (dp[e >> 2][qc][e & 3] - dl[qc]);
        pack8(dsf[qc], ds);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const Frag ta = lds_frag<T>(sT[st] + (16 * db + c) * TP, (8 * g) / E);
        acc[db][0] = mma16(acc[db][0], ta, dsf[0]);
        acc[db][1] = mma16(acc[db][1], ta, dsf[1]);
      }
    }
  };
  // The loads and stores run on every path (past the last tile they repeat it into the stage no
  // tile reads): with one skipped on some path, the compiler's waits in the loads covered loads
  // already stored.
  for (int t = 0; t < nt; t += 2) {
    K2_DQ_GLOAD(0, min(t + 1, nt - 1));
    tile(t, 0);
    K2_DQ_LSTORE(0, 1);
    __syncthreads();
    if (t + 1 >= nt) break;
    K2_DQ_GLOAD(0, min(t + 2, nt - 1));
    tile(t + 1, 1);
    K2_DQ_LSTORE(0, 0);
    __syncthreads();
  }
#undef K2_DQ_GLOAD
#undef K2_DQ_LSTORE
  // dQ^T block (db, qc): lane holds query q0 + 16 qc + c, head dims 16 db + 4 g + r
  if (active) {
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      const int qi = q0 + 16 * qc + c;
      if (qi >= L) continue;
      float* out = p.dq + (size_t)(b * L + qi) * p.lddq + head * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *(float4*)(out + 16 * db + 4 * g) = make_float4(acc[db][qc][0] * scale, acc[db][qc][1] * scale,
                                                        acc[db][qc][2] * scale, acc[db][qc][3] * scale);
    }
  }
}

template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_bwd_dkv_kernel(AttnBwdArgs p, float scale_log2, float scale, int nsplit) {
  typedef typename FragOf<T>::type Frag;
  constexpr int E = 16 / sizeof(T);
  constexpr int NC = HD / 32;
  constexpr int NDB = HD / 16;
  constexpr int RCH = HD / E;                // chunks per Q / dO row
  constexpr bool SWZ = sizeof(T) == 2 && RCH == 16;  // bf16 head_dim 128: swizzled rows (tile_chunk)
  constexpr int RP = SWZ ? RCH : RCH + 1;    // row pitch
  constexpr int TCH = 32 / E, TP = TCH + 1;  // chunks per Q^T / dO^T row (32 queries), row pitch
  constexpr int NQ = 32 * RCH / 256, NT = HD * TCH / 256;
  static_assert(NQ >= 1 && NT >= 1, "tile / thread mismatch");
  __shared__ uint4 sQ[2][32 * RP], sD[2][32 * RP], sQT[2][HD * TP], sDT[2][HD * TP];
  __shared__ float4 sL[2][8], sDl[2][8];
  K2_LDS_CHECK(sizeof(sQ) + sizeof(sD) + sizeof(sQT) + sizeof(sDT) + sizeof(sL) + sizeof(sDl), 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int G = p.nh / p.nkv;
  const int L = p.L, T_ = p.T;
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  // nsplit workgroups share a key block, each taking a contiguous share of its query tiles
  const int split = blockIdx.x % nsplit;
  const int k0 = (blockIdx.x / nsplit) * 128 + 32 * wave;
  const bool active = k0 < L;  // wave-uniform

  Frag kf[2][NC], vf[2][NC];
  bool kok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ki = k0 + 16 * j + c;
    kok[j] = ki < L && (ki >= T_ || !p.mask || p.mask[(size_t)b * T_ + ki] != 0);
    const size_t row = (size_t)(b * L + (ki < L ? ki : 0)) * ldk + kvh * HD + 8 * g;
#pragma unroll
    for (int kc = 0; kc < NC; ++kc) {
      kf[j][kc] = ki < L ? ld_frag<T>((const T*)p.k + row + 32 * kc) : zero_frag<T>();
      vf[j][kc] = ki < L ? ld_frag<T>((const T*)p.v + row + 32 * kc) : zero_frag<T>();
    }
  }
  f32x4 dk[NDB][2], dv[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db][0] = dk[db][1] = dv[db][0] = dv[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nt = (L + 31) / 32;
  // two register sets (tile loads run two tiles ahead of the products); macros rather than
  // lambdas keep both sets in registers. Tile u: query head kvh G + u / nt, queries 32 (u % nt) ..
  uint4 rq[2][NQ], rd[2][NQ], rqt[2][NT], rdt[2][NT];
  float rl[2] = {INFINITY, INFINITY}, rdl[2] = {0.0f, 0.0f};
  bool rok[2] = {false, false};
  // Tile loads are branch-free (buffer resources: rows past L read zero; every thread loads an lse /
  // Delta entry, the first 32 keep theirs), so the wait before a tile's LDS stores covers only that
  // tile's loads. Loaded through branches, the compiler waited for every load in flight there,
  // including the next tile's, and the loads were effectively one tile ahead instead of two.
  const size_t qspan = ((size_t)(L - 1) * ldq + HD) * sizeof(T);
  const size_t tspan = (size_t)HD * p.ldt * sizeof(T);  // a (batch, head) plane of Q^T / dO^T
#define K2_DKV_GLOAD(RS, u)                                                                        \
  do {                                                                                             \
    const int head_ = kvh * G + (u) / nt, t0_ = 32 * ((u) % nt);                                   \
    const rsrc_t qr_ = make_rsrc((const T*)p.q + (size_t)b * L * ldq + head_ * HD, qspan);         \
    const rsrc_t dr_ = make_rsrc((const T*)p.dout + (size_t)b * L * ldq + head_ * HD, qspan);      \
    const size_t tb_ = (size_t)(b * p.nh + head_) * HD * p.ldt;                                    \
    const rsrc_t qtr_ = make_rsrc((const T*)p.qt + tb_, tspan);                                    \
    const rsrc_t dtr_ = make_rsrc((const T*)p.dot + tb_, tspan);                                   \
    _Pragma("unroll") for (int i = 0; i < NQ; ++i) {                                               \
      const int ch_ = tid + 256 * i, row_ = ch_ / RCH, cc_ = ch_ % RCH, q_ = t0_ + row_;            \
      const uint32_t off_ = q_ < L ? (uint32_t)(q_ * ldq + cc_ * E) * (uint32_t)sizeof(T) : kOOB;  \
      rq[RS][i] = bload(qr_, off_);                                                                \
      rd[RS][i] = bload(dr_, off_);                                                                \
    }                                                                                              \
    /* Q^T, dO^T: zero past L (written so by the transposes) */                                    \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                               \
      const int ch_ = tid + 256 * i, d_ = ch_ / TCH, cc_ = ch_ % TCH;                               \
      const uint32_t off_ = (uint32_t)(d_ * p.ldt + t0_ + cc_ * E) * (uint32_t)sizeof(T);          \
      rqt[RS][i] = bload(qtr_, off_);                                                              \
      rdt[RS][i] = bload(dtr_, off_);                                                              \
    }                                                                                              \
    {  /* raw values; queries past L get lse +inf and Delta 0 at the LDS store */                  \
      const int q_ = t0_ + (tid & 31);                                                             \
      const size_t ri_ = ((size_t)b * p.nh + head_) * L + (q_ < L ? q_ : L - 1);                   \
      rl[RS] = p.lse[ri_];                                                                         \
      rdl[RS] = p.delta[ri_];                                                                      \
      rok[RS] = q_ < L;                                                                            \
    }                                                                                              \
  } while (0)
#define K2_DKV_LSTORE(RS, ST)                                                                      \
  do {                                                                                             \
    _Pragma("unroll") for (int i = 0; i < NQ; ++i) {                                               \
      const int ch_ = tid + 256 * i, row_ = ch_ / RCH, cc_ = ch_ % RCH;                             \
      sQ[ST][row_ * RP + tile_chunk<SWZ>(row_, cc_)] = rq[RS][i];                                  \
      sD[ST][row_ * RP + tile_chunk<SWZ>(row_, cc_)] = rd[RS][i];                                  \
    }                                                                                              \
    _Pragma("unroll") for (int i = 0; i < NT; ++i) {                                               \
      const int ch_ = tid + 256 * i, d_ = ch_ / TCH, cc_ = ch_ % TCH;                               \
      sQT[ST][d_ * TP + cc_] = rqt[RS][i];                                                         \
      sDT[ST][d_ * TP + cc_] = rdt[RS][i];                                                         \
    }                                                                                              \
    if (tid < 32) {                                                                                \
      reinterpret_cast<float*>(sL[ST])[tid] = rok[RS] ? rl[RS] : INFINITY;                         \
      reinterpret_cast<float*>(sDl[ST])[tid] = rok[RS] ? rdl[RS] : 0.0f;                           \
    }                                                                                              \
  } while (0)

  const int nu = G * nt;
  const int u0 = split * nu / nsplit, u1 = (split + 1) * nu / nsplit;  // u0 < u1: nu >= nsplit
  // Tile u's loads go out at the start of tile u - 2 and its LDS stores at the start of tile u - 1,
  // so the wait before a store covers loads two tiles old while the next tile's stay in flight. The
  // loads are issued on every path (past the last tile they reload it, unused): with a load skipped
  // on some path, the compiler's wait before a store had to cover every load in flight.
  const int ulast = u1 - 1;
  K2_DKV_GLOAD(0, u0);
  K2_DKV_GLOAD(1, min(u0 + 1, ulast));
  K2_DKV_LSTORE(0, 0);
  K2_DKV_GLOAD(0, min(u0 + 2, ulast));
  __syncthreads();
  // One tile, ordered so that the matrix cores have independent work during the vector steps:
  // S = K Q^T; dP = V dO^T with P = exp2(S log2(e)/sqrt(hd) - lse) computed alongside; dV += P^T dO
  // with dS = P (dP - Delta) computed alongside; dK += dS^T Q.
  // The tile's 4 NC + 2 NDB LDS fragments (Q rows, dO rows, dO^T rows, Q^T rows, in that order)
  // stream through a ring RA reads ahead of the matrix-core step that takes them, across the phase
  // boundaries. With one wave per SIMD nothing else hides an LDS read's latency: read one step
  // ahead, as the compiler scheduled it, the pass kept the matrix cores 25 % busy.
  constexpr int NF = 4 * NC + 2 * NDB, RA = sizeof(T) == 2 ? 6 : 2;  // float32 fragments take 8 registers
  const int qro[2] = {perm32(0, c), perm32(1, c)};
  auto tile = [&](int u, int st) {
    if (active) {
      // queries 8g + 4qb + r of the tile (lse +inf past L, so their P is 0): float4 2g + qb
      float ql[8], qd[8];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float4 a = sL[st][2 * g + qb], d4 = sDl[st][2 * g + qb];
        ql[4 * qb] = a.x; ql[4 * qb + 1] = a.y; ql[4 * qb + 2] = a.z; ql[4 * qb + 3] = a.w;
        qd[4 * qb] = d4.x; qd[4 * qb + 1] = d4.y; qd[4 * qb + 2] = d4.z; qd[4 * qb + 3] = d4.w;
      }
      // fragment f of the tile (f is a compile-time constant at every call)
      auto frag = [&](int f) -> Frag {
        if (f < 2 * NC) {
          const int qb = f / NC, kc = f % NC;
          return lds_frag<T>(sQ[st] + qro[qb] * RP, tile_chunk<SWZ>(qro[qb], (32 * kc + 8 * g) / E));
        }
        if (f < 4 * NC) {
          const int qb = (f - 2 * NC) / NC, kc = (f - 2 * NC) % NC;
          return lds_frag<T>(sD[st] + qro[qb] * RP, tile_chunk<SWZ>(qro[qb], (32 * kc + 8 * g) / E));
        }
        if (f < 4 * NC + NDB) return lds_frag<T>(sDT[st] + (16 * (f - 4 * NC) + c) * TP, (8 * g) / E);
        return lds_frag<T>(sQT[st] + (16 * (f - 4 * NC - NDB) + c) * TP, (8 * g) / E);
      };
      f32x4 s[2][2], dp[2][2];
      float pv[2][8];  // P of key block j: entry 4 qb + r
      float dsv[2][8];
      Frag pf[2], dsf[2];
      Frag ring[RA + 1];
#pragma unroll
      for (int f = 0; f < RA; ++f) ring[f] = frag(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + RA < NF) ring[(f + RA) % (RA + 1)] = frag(f + RA);
        const Frag a = ring[f % (RA + 1)];
        if (f < 2 * NC) {  // S
          const int qb = f / NC, kc = f % NC;
#pragma unroll
          for (int j = 0; j < 2; ++j) s[qb][j] = mma16(kc ? s[qb][j] : f32x4{0.f, 0.f, 0.f, 0.f}, a, kf[j][kc]);
        } else if (f < 4 * NC) {  // dP, with 8 / NC exponentials of query block qb per step
          const int qb = (f - 2 * NC) / NC, kc = (f - 2 * NC) % NC;
#pragma unroll
          for (int j = 0; j < 2; ++j) dp[qb][j] = mma16(kc ? dp[qb][j] : f32x4{0.f, 0.f, 0.f, 0.f}, a, vf[j][kc]);
#pragma unroll
          for (int x = kc * 8 / NC; x < (kc + 1) * 8 / NC; ++x) {
            const int j = x >> 2, r = x & 3;
            pv[j][4 * qb + r] = kok[j] ? __builtin_amdgcn_exp2f(fmaf(s[qb][j][r], scale_log2, -ql[4 * qb + r])) : 0.0f;
          }
          if (f == 4 * NC - 1) {
            pack8(pf[0], pv[0]);
            pack8(pf[1], pv[1]);
          }
        } else if (f < 4 * NC + NDB) {  // dV, with 16 / NDB entries of dS per step
          const int db = f - 4 * NC;
#pragma unroll
          for (int j = 0; j < 2; ++j) dv[db][j] = mma16(dv[db][j], a, pf[j]);
#pragma unroll
          for (int x = db * 16 / NDB; x < (db + 1) * 16 / NDB; ++x) {
            const int j = x >> 3, e = x & 7;
            dsv[j][e] = pv[j][e] * (dp[e >> 2][j][e & 3] - qd[e]);
          }
          if (db == NDB - 1) {
            pack8(dsf[0], dsv[0]);
            pack8(dsf[1], dsv[1]);
          }
        } else {  // dK
          const int db = f - 4 * NC - NDB;
#pragma unroll
          for (int j = 0; j < 2; ++j) dk[db][j] = mma16(dk[db][j], a, dsf[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int u = u0; u < u1; u += 2) {
    if (u + 1 < u1) K2_DKV_LSTORE(1, 1);  // stage 1 was last read by tile u - 1 (before the barrier)
    K2_DKV_GLOAD(1, min(u + 3, ulast));
    tile(u, 0);
    __syncthreads();
    if (u + 1 >= u1) break;
    if (u + 2 < u1) K2_DKV_LSTORE(0, 0);
    K2_DKV_GLOAD(0, min(u + 4, ulast));
    tile(u + 1, 1);
    __syncthreads();
  }
#undef K2_DKV_GLOAD
#undef K2_DKV_LSTORE
  // dK^T / dV^T block (db, j): lane holds key k0 + 16 j + c, head dims 16 db + 4 g + r
  if (active && nsplit > 1) {  // partial sums: dK into plane 2 split, dV into plane 2 split + 1
    const size_t plane = (size_t)p.B * L * ldk;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ki = k0 + 16 * j + c;
      if (ki >= L) continue;
      float* ko = p.dkv_part + 2 * split * plane + (size_t)(b * L + ki) * ldk + kvh * HD;
      float* vo = ko + plane;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        *(float4*)(ko + 16 * db + 4 * g) = make_float4(dk[db][j][0] * scale, dk[db][j][1] * scale,
                                                       dk[db][j][2] * scale, dk[db][j][3] * scale);
        *(float4*)(vo + 16 * db + 4 * g) = make_float4(dv[db][j][0], dv[db][j][1], dv[db][j][2], dv[db][j][3]);
      }
    }
  } else if (active) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ki = k0 + 16 * j + c;
      if (ki >= L) continue;
      float* ko = p.dk + (size_t)(b * L + ki) * p.lddk + kvh * HD;
      T* vo = (T*)p.dv + (size_t)(b * L + ki) * p.lddv + kvh * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        *(float4*)(ko + 16 * db + 4 * g) = make_float4(dk[db][j][0] * scale, dk[db][j][1] * scale,
                                                       dk[db][j][2] * scale, dk[db][j][3] * scale);
#pragma unroll
        for (int r = 0; r < 4; ++r) vo[16 * db + 4 * g + r] = (T)dv[db][j][r];
      }
    }
  }
}

// dK = dK part 0 + dK part 1 (float32), dV = T(dV part 0 + dV part 1); planes of `plane` floats in
// the order dK0, dV0, dK1, dV1; rows of nk columns.
template <typename T>
__global__ void __launch_bounds__(256) dkv_combine_kernel(const float* __restrict__ part, size_t n4, int nk, size_t plane,
                                                          float* __restrict__ dk, int lddk, T* __restrict__ dv, int lddv) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const size_t e = 4 * i, m = e / nk, c = e - m * nk;
    const float4 k0 = *(const float4*)(part + e), v0 = *(const float4*)(part + plane + e);
    const float4 k1 = *(const float4*)(part + 2 * plane + e), v1 = *(const float4*)(part + 3 * plane + e);
    *(float4*)(dk + m * lddk + c) = make_float4(k0.x + k1.x, k0.y + k1.y, k0.z + k1.z, k0.w + k1.w);
    T* o = dv + m * lddv + c;
    o[0] = (T)(v0.x + v1.x);
    o[1] = (T)(v0.y + v1.y);
    o[2] = (T)(v0.z + v1.z);
    o[3] = (T)(v0.w + v1.w);
  }
}

// compute units of the current device
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

template <typename T, int HD, int G>
static hipError_t attn_bwd_t(const AttnBwdArgs& p, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)HD);
  const float scale_log2 = 1.4426950408889634f * scale;
  constexpr int QW = 32 * (4 / G);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD, G>), dim3((p.L + QW - 1) / QW, p.nkv, p.B), dim3(256), 0, s, p,
                     scale_log2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK/dV: one workgroup per compute unit (registers). Its grid of key blocks often leaves the last
  // round part-empty (block1024: 864 workgroups = 3.4 rounds of 256); splitting each key block's
  // query tiles over two workgroups fills the rounds better (6.75 of 7) at the price of one pass
  // summing the float32 partials.
  const int W = (p.L + 127) / 128 * p.nkv * p.B, ncu = cu_count();
  const double e1 = (double)W / ((double)((W + ncu - 1) / ncu) * ncu);
  const double e2 = (double)(2 * W) / ((double)((2 * W + ncu - 1) / ncu) * ncu);
  const int nsplit = p.dkv_part && G * ((p.L + 31) / 32) >= 2 && e2 > e1 ? 2 : 1;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, HD>), dim3((p.L + 127) / 128 * nsplit, p.nkv, p.B), dim3(256), 0, s, p,
                     scale_log2, scale, nsplit);
  e = hipGetLastError();
  if (e != hipSuccess || nsplit == 1) return e;
  const size_t n4 = (size_t)p.B * p.L * p.nkv * HD / 4;
  const int blocks = (int)((n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192);
  hipLaunchKernelGGL(dkv_combine_kernel<T>, dim3(blocks), dim3(256), 0, s, (const float*)p.dkv_part, n4,
                     p.nkv * HD, (size_t)p.B * p.L * p.nkv * HD, p.dk, p.lddk, (T*)p.dv, p.lddv);
  return hipGetLastError();
}

template <typename T, int HD>
static hipError_t attn_bwd_g(const AttnBwdArgs& p, hipStream_t s) {
  const int G = p.nh / p.nkv;
  if (G == 4) return attn_bwd_t<T, HD, 4>(p, s);
  if (G == 2) return attn_bwd_t<T, HD, 2>(p, s);
  if (G == 1) return attn_bwd_t<T, HD, 1>(p, s);
  return hipErrorInvalidValue;
}

hipError_t attention_backward(int dt, const AttnBwdArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.L <= 0) return hipSuccess;
  // the K^T, Q^T and dO^T rows hold 32-key / 32-query tiles up to the last one
  if (p.nh % p.nkv || p.ldt < (p.L + 31) / 32 * 32 || p.ldt % 8 || p.T > kBwdTextTiles * 32) return hipErrorInvalidValue;
  if (p.hd == 128) return dt == DT_BF16 ? attn_bwd_g<bf16, 128>(p, s) : attn_bwd_g<float, 128>(p, s);
  if (p.hd == 64) return dt == DT_BF16 ? attn_bwd_g<bf16, 64>(p, s) : attn_bwd_g<float, 64>(p, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// q/k norm + RoPE backward per (row, head): with dr the gradient of the rotated, normed head,
// dn = R(-phi) dr (the rotation's transpose), g = dn (1 + w), dx = r g - x r^3 sum(g x) / HD for
// the raw projection x, r = 1/sqrt(mean(x^2) + eps); dx goes out in the operand dtype. Partial sums
// of dn x r over the workgroup's items give the norm weight's gradient (part[block][HD]).
// HD/8 threads per item (8 head dims, 4 rotation pairs each); items in a grid-stride loop.
// ---------------------------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(256) qknorm_bwd_kernel(QkNormBwdArgs p) {
  constexpr int TPI = HD / 8, IPB = 256 / TPI;  // threads per item, items per pass of a block
  __shared__ float red[IPB][HD];
  K2_LDS_CHECK(sizeof(red), 1);
  const int ch = threadIdx.x % TPI, slot = threadIdx.x / TPI;
  float wd[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) wd[e] = 0.0f;
  float mult[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mult[e] = 1.0f + (p.w ? p.w[8 * ch + e] : 0.0f);
  const long nitems = (long)p.M * p.heads;
  for (long item = (long)blockIdx.x * IPB + slot; item < nitems + 0; item += (long)gridDim.x * IPB) {
    const int m = (int)(item / p.heads), h = (int)(item - (long)m * p.heads);
    const float* dr = p.dr + (size_t)m * p.lddr + h * HD + 8 * ch;
    const float* x = p.x + (size_t)m * p.ldx + h * HD + 8 * ch;
    float dn[8], xv[8];
    const float4 d0 = *(const float4*)dr, d1 = *(const float4*)(dr + 4);
    const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
    dn[0] = d0.x; dn[1] = d0.y; dn[2] = d0.z; dn[3] = d0.w; dn[4] = d1.x; dn[5] = d1.y; dn[6] = d1.z; dn[7] = d1.w;
    xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w; xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
    if (p.rc) {
      const int l = m % p.L;
      const float* cs = p.rc + (size_t)l * (HD / 2) + 4 * ch;
      const float* sn = p.rs + (size_t)l * (HD / 2) + 4 * ch;
#pragma unroll
      for (int q = 0; q < 4; ++q) {  // pair (2q, 2q + 1) turned back by its angle
        const float a = dn[2 * q], bb = dn[2 * q + 1], co = cs[q], si = sn[q];
        dn[2 * q] = a * co + bb * si;
        dn[2 * q + 1] = bb * co - a * si;
      }
    }
    float ss = 0.0f, dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += xv[e] * xv[e];
      dot += dn[e] * mult[e] * xv[e];
    }
    ss = group_sum<TPI>(ss);
    dot = group_sum<TPI>(dot);
    const float r = rsqrtf(ss / (float)HD + p.eps);
    const float k3 = r * r * r * dot / (float)HD;
    T* out = (T*)p.dx + (size_t)m * p.lddx + h * HD + 8 * ch;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      out[e] = (T)(r * dn[e] * mult[e] - xv[e] * k3);
      wd[e] += dn[e] * xv[e] * r;
    }
  }
  if (!p.part) return;  // uniform
#pragma unroll
  for (int e = 0; e < 8; ++e) red[slot][8 * ch + e] = wd[e];
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += 256) {
    float acc = 0.0f;
    for (int i = 0; i < IPB; ++i) acc += red[i][d];
    p.part[(size_t)blockIdx.x * HD + d] = acc;
  }
}

hipError_t qknorm_bwd(int dt, const QkNormBwdArgs& p, int blocks, hipStream_t s) {
  if (p.M <= 0 || p.heads <= 0) return hipSuccess;
  if (p.hd == 128 && dt == DT_BF16)
    hipLaunchKernelGGL((qknorm_bwd_kernel<bf16, 128>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 128)
    hipLaunchKernelGGL((qknorm_bwd_kernel<float, 128>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 64 && dt == DT_BF16)
    hipLaunchKernelGGL((qknorm_bwd_kernel<bf16, 64>), dim3(blocks), dim3(256), 0, s, p);
  else if (p.hd == 64)
    hipLaunchKernelGGL((qknorm_bwd_kernel<float, 64>), dim3(blocks), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// out[gr * ldo + j] = sum_{c < nc} part[(gr * nc + c) * ldp + j] for gr < G, j < ncols
// ---------------------------------------------------------------------------------------------
// 256 threads = 64 columns x 4 chunk lanes; each thread keeps 4 independent sums so that many loads
// are in flight, then the 4 chunk lanes meet in LDS
__device__ __forceinline__ void reduce_rows_block(const float* __restrict__ part, int nc, int ncols, int ldp,
                                                  float* __restrict__ out, int ldo, int gr, int cb) {
  __shared__ float red[4][64];
  K2_LDS_CHECK(sizeof(red), 1);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int j = cb * 64 + tx;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  if (j < ncols) {
    const float* pp = part + (size_t)gr * nc * ldp + j;
    int cc = ty;
    for (; cc + 12 < nc; cc += 16) {
      a0 += pp[(size_t)cc * ldp];
      a1 += pp[(size_t)(cc + 4) * ldp];
      a2 += pp[(size_t)(cc + 8) * ldp];
      a3 += pp[(size_t)(cc + 12) * ldp];
    }
    for (; cc < nc; cc += 4) a0 += pp[(size_t)cc * ldp];
  }
  red[ty][tx] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  if (ty == 0 && j < ncols) out[(size_t)gr * ldo + j] = (red[0][tx] + red[1][tx]) + (red[2][tx] + red[3][tx]);
}

__global__ void __launch_bounds__(256) reduce_rows_kernel(const float* __restrict__ part, int G, int nc, int ncols,
                                                          int ldp, float* __restrict__ out, int ldo) {
  reduce_rows_block(part, nc, ncols, ldp, out, ldo, blockIdx.y, blockIdx.x);
}

// several independent reductions in one launch: blockIdx.z picks the job; blocks past a job's
// columns or groups leave at once (the whole block, before its barrier)
__global__ void __launch_bounds__(256) reduce_rows_multi_kernel(ReduceJobs jobs) {
  const ReduceJob& jb = jobs.job[blockIdx.z];
  if ((int)blockIdx.x * 64 >= jb.ncols || (int)blockIdx.y >= jb.G) return;
  reduce_rows_block(jb.part, jb.nc, jb.ncols, jb.ldp, jb.out, jb.ldo, blockIdx.y, blockIdx.x);
}

hipError_t reduce_rows(const float* part, int G, int nc, int ncols, int ldp, float* out, int ldo, hipStream_t s) {
  if (G <= 0 || ncols <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((ncols + 63) / 64, G), dim3(256), 0, s, part, G, nc, ncols, ldp, out,
                     ldo);
  return hipGetLastError();
}

hipError_t reduce_rows_multi(const ReduceJobs& jobs, hipStream_t s) {
  if (jobs.n <= 0) return hipSuccess;
  if (jobs.n > kMaxReduceJobs) return hipErrorInvalidValue;
  int gx = 1, gy = 1;
  for (int i = 0; i < jobs.n; ++i) {
    gx = std::max(gx, (jobs.job[i].ncols + 63) / 64);
    gy = std::max(gy, jobs.job[i].G);
  }
  hipLaunchKernelGGL(reduce_rows_multi_kernel, dim3(gx, gy, jobs.n), dim3(256), 0, s, jobs);
  return hipGetLastError();
}

}  // namespace k2
