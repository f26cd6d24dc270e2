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
//   attn_bwd_dq    — dQ = dS K / sqrt(hd), one wave per 16 queries of one head
//   attn_bwd_dkv   — dK = dS^T Q / sqrt(hd) and dV = P^T dO over the query heads of a kv head,
//                    one wave per 16 keys
//   qknorm_bwd     — the RoPE rotation's transpose, then the per-head RMSNorm backward
//   reduce_rows    — sums of the per-chunk partials
//
// Attention backward, with P = softmax(S), S = Q K^T / sqrt(hd) under the key mask, O = P V:
// dV = P^T dO, dP = dO V^T, dS = P (dP - Delta), Delta = rowsum(dO * O); P is recomputed from the
// forward's per-row log-sum-exp. Both kernels use the 16x16 matrix-core block of k2_device.h for
// bf16 and float32 operands; fragments load straight from memory (no LDS), and the permuted row
// order of the forward's float32 kernel (accumulator row 4g + r of 16-row block kb is index
// 8g + 4kb + r) makes the probabilities a lane holds the operand of the next product.
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

hipError_t transpose(int dt, const TransposeArgs& p, hipStream_t s) {
  if (p.R <= 0 || p.C <= 0 || p.Z <= 0) return hipSuccess;
  if (p.Rpad < p.R || p.ldd < p.Rpad || p.zdiv <= 0) return hipErrorInvalidValue;
  dim3 grid((p.C + 63) / 64, (p.Rpad + 63) / 64, p.Z);
  if (dt == DT_BF16)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, p);
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

hipError_t swiglu_bwd(int dt, const float* da, const float* gt, const float* up, int M, int I, void* dgu,
                      hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const size_t n = (size_t)M * I;
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
__global__ void __launch_bounds__(256) norm_bwd_kernel(NormBwdArgs p) {
  constexpr int CACHE = 8;
  __shared__ float red[2][4];
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
    const int cc = tid + u * 256;
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
    float4 xv[CACHE], dv[CACHE];
    float ss = 0.0f, dot = 0.0f;
#pragma unroll
    for (int u = 0; u < CACHE; ++u) {
      const int cc = tid + u * 256;
      xv[u] = dv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (cc < H4) {
        xv[u] = x4[cc];
        dv[u] = d4[cc];
        ss += xv[u].x * xv[u].x + xv[u].y * xv[u].y + xv[u].z * xv[u].z + xv[u].w * xv[u].w;
        // g = dout (1 + sc) (1 + w)
        dot += dv[u].x * ms[u].x * mw[u].x * xv[u].x + dv[u].y * ms[u].y * mw[u].y * xv[u].y +
               dv[u].z * ms[u].z * mw[u].z * xv[u].z + dv[u].w * ms[u].w * mw[u].w * xv[u].w;
      }
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    if ((tid & 63) == 0) {
      red[0][wv] = ss;
      red[1][wv] = dot;
    }
    __syncthreads();
    ss = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    dot = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    __syncthreads();
    const float r = rsqrtf(ss / (float)p.H + p.eps);
    const float k3 = r * r * r * dot / (float)p.H;
    const float4* res4 = p.dres ? (const float4*)(p.dres + row * p.H) : nullptr;
    float4* o4 = (float4*)(p.dx + row * p.H);
#pragma unroll
    for (int u = 0; u < CACHE; ++u) {
      const int cc = tid + u * 256;
      if (cc >= H4) continue;
      const float4 x = xv[u], d = dv[u], m1 = ms[u], m2 = mw[u];
      float4 res = res4 ? res4[cc] : make_float4(0.f, 0.f, 0.f, 0.f);
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
    const int cc = tid + u * 256;
    if (cc >= H4) continue;
    if (p.pw) ((float4*)(p.pw + (size_t)chunk * p.H))[cc] = pw[u];
    if (p.psc) ((float4*)(p.psc + (size_t)chunk * p.H))[cc] = psc[u];
    if (p.psh) ((float4*)(p.psh + (size_t)chunk * p.H))[cc] = psh[u];
  }
}

hipError_t norm_bwd(const NormBwdArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.L <= 0) return hipSuccess;
  if (p.H % 4 || p.H > 8 * 256 * 4 || p.RC <= 0 || p.ncb != (p.L + p.RC - 1) / p.RC) return hipErrorInvalidValue;
  hipLaunchKernelGGL(norm_bwd_kernel, dim3(p.B * p.ncb), dim3(256), 0, s, p);
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
  float dsum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float s = sigm((float)g[e]), ov = (float)o[e], d = dog[e];
    const T dt = (T)(d * s);
    dout[e] = dt;
    dg[e] = (T)(d * ov * s * (1.0f - s));
    dsum += (float)dt * ov;
  }
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
// Attention backward, dQ: one wave per (batch row, query head, 16 queries), 4 waves per
// workgroup on consecutive query blocks. Per 32-key tile (two 16-key blocks kb):
//   S^T = K Q^T     A: K rows (keys permuted by perm32), B: Q^T (query column, 8 head dims)
//   P^T = exp2(S^T scale_log2 - lse2[q]) on allowed keys
//   dP^T = V dO^T   A: V rows (same permutation), B: dO^T
//   dS^T = P^T (dP^T - Delta[q])
//   dQ^T += K^T dS^T A: K^T rows (head dim, 8 consecutive keys), B: dS^T from registers
// Lane l holds query column l % 16; lane group g = l / 16 holds keys 8g .. 8g + 7 of the tile.
// ---------------------------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(AttnBwdArgs p, float scale_log2, float scale) {
  typedef typename FragOf<T>::type Frag;
  constexpr int NC = HD / 32;  // 32-wide head-dim chunks
  constexpr int NDB = HD / 16; // 16-row head-dim blocks of dQ^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, head = blockIdx.y;
  const int kvh = head / (p.nh / p.nkv);
  const int L = p.L, T_ = p.T;
  const int q0 = (blockIdx.x * 4 + wave) * 16;
  if (q0 >= L) return;  // no barriers in this kernel
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const int qi = q0 + c;
  const bool qok = qi < L;
  const T* qrow = (const T*)p.q + (size_t)(b * L + (qok ? qi : 0)) * ldq + head * HD;
  const T* drow = (const T*)p.dout + (size_t)(b * L + (qok ? qi : 0)) * ldq + head * HD;
  Frag qf[NC], df[NC];
#pragma unroll
  for (int kc = 0; kc < NC; ++kc) {
    qf[kc] = qok ? ld_frag<T>(qrow + 32 * kc + 8 * g) : zero_frag<T>();
    df[kc] = qok ? ld_frag<T>(drow + 32 * kc + 8 * g) : zero_frag<T>();
  }
  const size_t rowstat = ((size_t)b * p.nh + head) * L + (qok ? qi : 0);
  const float lse = qok ? p.lse[rowstat] : INFINITY;
  const float delta = qok ? p.delta[rowstat] : 0.0f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const T* kbase = (const T*)p.k + (size_t)b * L * ldk + kvh * HD;
  const T* vbase = (const T*)p.v + (size_t)b * L * ldk + kvh * HD;
  const T* ktbase = (const T*)p.kt + (size_t)(b * p.nkv + kvh) * HD * p.ldt;
  for (int t0 = 0; t0 < L; t0 += 32) {
    f32x4 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = t0 + perm32(kb, c);  // this lane's A row
      const bool kok = key < L;
      const T* kr = kbase + (size_t)(kok ? key : 0) * ldk + 8 * g;
      const T* vr = vbase + (size_t)(kok ? key : 0) * ldk + 8 * g;
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        const Frag ka = kok ? ld_frag<T>(kr + 32 * kc) : zero_frag<T>();
        const Frag va = kok ? ld_frag<T>(vr + 32 * kc) : zero_frag<T>();
        s[kb] = mma16(s[kb], ka, qf[kc]);
        dp[kb] = mma16(dp[kb], va, df[kc]);
      }
    }
    // accumulator row 4g + r of block kb is key t0 + 8g + 4kb + r, column c is query qi
    float ds[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t0 + 8 * g + 4 * kb + r;
        const bool ok = key < L && (key >= T_ || !p.mask || p.mask[(size_t)b * T_ + key] != 0);
        const float pr = ok ? exp2f(s[kb][r] * scale_log2 - lse) : 0.0f;
        ds[4 * kb + r] = pr * (dp[kb][r] - delta);
      }
    Frag dsf;
    pack8(dsf, ds);
    const int kn = min(8, L - (t0 + 8 * g));  // valid keys among this lane group's 8
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const T* ktr = ktbase + (size_t)(16 * db + c) * p.ldt + t0 + 8 * g;
      const Frag ka = kn > 0 ? ld_frag_n<T>(ktr, kn) : zero_frag<T>();
      acc[db] = mma16(acc[db], ka, dsf);
    }
  }
  // dQ^T block db: lane holds query column c, head dims 16 db + 4 g + r
  if (qok) {
    float* out = p.dq + (size_t)(b * L + qi) * p.lddq + head * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *(float4*)(out + 16 * db + 4 * g) =
          make_float4(acc[db][0] * scale, acc[db][1] * scale, acc[db][2] * scale, acc[db][3] * scale);
  }
}

// ---------------------------------------------------------------------------------------------
// Attention backward, dK and dV: one wave per (batch row, kv head, 16 keys), 4 waves per workgroup
// on consecutive key blocks; each wave runs over the G query heads of its kv head and all query
// tiles. Per 32-query tile (two 16-query blocks qb):
//   S = Q K^T       A: Q rows (queries permuted by perm32), B: K^T (key column, 8 head dims)
//   P = exp2(S scale_log2 - lse2[q]) on allowed keys
//   dP = dO V^T     A: dO rows (same permutation), B: V^T (key column)
//   dS = P (dP - Delta[q])
//   dV^T += dO^T P  A: dO^T rows (head dim, 8 consecutive queries), B: P from registers
//   dK^T += Q^T dS  A: Q^T rows, B: dS from registers
// ---------------------------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(256) attn_bwd_dkv_kernel(AttnBwdArgs p, float scale_log2, float scale) {
  typedef typename FragOf<T>::type Frag;
  constexpr int NC = HD / 32;
  constexpr int NDB = HD / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int G = p.nh / p.nkv;
  const int L = p.L, T_ = p.T;
  const int k0 = (blockIdx.x * 4 + wave) * 16;
  if (k0 >= L) return;  // no barriers in this kernel
  const int ldq = p.nh * HD, ldk = p.nkv * HD;
  const int ki = k0 + c;
  const bool kok = ki < L && (ki >= T_ || !p.mask || p.mask[(size_t)b * T_ + ki] != 0);
  const T* krow = (const T*)p.k + (size_t)(b * L + (ki < L ? ki : 0)) * ldk + kvh * HD;
  const T* vrow = (const T*)p.v + (size_t)(b * L + (ki < L ? ki : 0)) * ldk + kvh * HD;
  Frag kf[NC], vf[NC];
#pragma unroll
  for (int kc = 0; kc < NC; ++kc) {
    kf[kc] = ki < L ? ld_frag<T>(krow + 32 * kc + 8 * g) : zero_frag<T>();
    vf[kc] = ki < L ? ld_frag<T>(vrow + 32 * kc + 8 * g) : zero_frag<T>();
  }
  f32x4 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < G; ++hh) {
    const int head = kvh * G + hh;
    const T* qbase = (const T*)p.q + (size_t)b * L * ldq + head * HD;
    const T* dbase = (const T*)p.dout + (size_t)b * L * ldq + head * HD;
    const T* qtbase = (const T*)p.qt + (size_t)(b * p.nh + head) * HD * p.ldt;
    const T* dtbase = (const T*)p.dot + (size_t)(b * p.nh + head) * HD * p.ldt;
    const float* lse = p.lse + ((size_t)b * p.nh + head) * L;
    const float* dl = p.delta + ((size_t)b * p.nh + head) * L;
    for (int t0 = 0; t0 < L; t0 += 32) {
      f32x4 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = dp[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int q = t0 + perm32(qb, c);  // this lane's A row
        const bool qok = q < L;
        const T* qr = qbase + (size_t)(qok ? q : 0) * ldq + 8 * g;
        const T* dr = dbase + (size_t)(qok ? q : 0) * ldq + 8 * g;
#pragma unroll
        for (int kc = 0; kc < NC; ++kc) {
          const Frag qa = qok ? ld_frag<T>(qr + 32 * kc) : zero_frag<T>();
          const Frag da = qok ? ld_frag<T>(dr + 32 * kc) : zero_frag<T>();
          s[qb] = mma16(s[qb], qa, kf[kc]);
          dp[qb] = mma16(dp[qb], da, vf[kc]);
        }
      }
      // accumulator row 4g + r of block qb is query t0 + 8g + 4qb + r, column c is key ki
      float pv[8], ds[8];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = t0 + 8 * g + 4 * qb + r;
          float pr = 0.0f, dd = 0.0f;
          if (kok && q < L) {
            pr = exp2f(s[qb][r] * scale_log2 - lse[q]);
            dd = pr * (dp[qb][r] - dl[q]);
          }
          pv[4 * qb + r] = pr;
          ds[4 * qb + r] = dd;
        }
      Frag pf, dsf;
      pack8(pf, pv);
      pack8(dsf, ds);
      const int qn = min(8, L - (t0 + 8 * g));  // valid queries among this lane group's 8
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const size_t off = (size_t)(16 * db + c) * p.ldt + t0 + 8 * g;
        const Frag da = qn > 0 ? ld_frag_n<T>(dtbase + off, qn) : zero_frag<T>();
        const Frag qa = qn > 0 ? ld_frag_n<T>(qtbase + off, qn) : zero_frag<T>();
        dv[db] = mma16(dv[db], da, pf);
        dk[db] = mma16(dk[db], qa, dsf);
      }
    }
  }
  // dK^T / dV^T block db: lane holds key column c, head dims 16 db + 4 g + r
  if (ki < L) {
    float* ko = p.dk + (size_t)(b * L + ki) * p.lddk + kvh * HD;
    T* vo = (T*)p.dv + (size_t)(b * L + ki) * p.lddv + kvh * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      *(float4*)(ko + 16 * db + 4 * g) =
          make_float4(dk[db][0] * scale, dk[db][1] * scale, dk[db][2] * scale, dk[db][3] * scale);
#pragma unroll
      for (int r = 0; r < 4; ++r) vo[16 * db + 4 * g + r] = (T)dv[db][r];
    }
  }
}

template <typename T, int HD>
static hipError_t attn_bwd_t(const AttnBwdArgs& p, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)HD);
  const float scale_log2 = 1.4426950408889634f * scale;
  const int nb = (p.L + 63) / 64;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, HD>), dim3(nb, p.nh, p.B), dim3(256), 0, s, p, scale_log2, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<T, HD>), dim3(nb, p.nkv, p.B), dim3(256), 0, s, p, scale_log2, scale);
  return hipGetLastError();
}

hipError_t attention_backward(int dt, const AttnBwdArgs& p, hipStream_t s) {
  if (p.B <= 0 || p.L <= 0) return hipSuccess;
  if (p.nh % p.nkv || p.ldt < p.L || p.ldt % 8) return hipErrorInvalidValue;
  if (p.hd == 128) return dt == DT_BF16 ? attn_bwd_t<bf16, 128>(p, s) : attn_bwd_t<float, 128>(p, s);
  if (p.hd == 64) return dt == DT_BF16 ? attn_bwd_t<bf16, 64>(p, s) : attn_bwd_t<float, 64>(p, s);
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
__global__ void __launch_bounds__(256) reduce_rows_kernel(const float* __restrict__ part, int G, int nc, int ncols,
                                                          int ldp, float* __restrict__ out, int ldo) {
  __shared__ float red[4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + tx;
  const int gr = blockIdx.y;
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

hipError_t reduce_rows(const float* part, int G, int nc, int ncols, int ldp, float* out, int ldo, hipStream_t s) {
  if (G <= 0 || ncols <= 0) return hipSuccess;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((ncols + 63) / 64, G), dim3(256), 0, s, part, G, nc, ncols, ldp, out,
                     ldo);
  return hipGetLastError();
}

}  // namespace k2
