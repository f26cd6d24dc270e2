// Internal launcher interface between the C ABI (k2_api.cpp) and the kernel translation units.
// Plain structs of device pointers and sizes; each launcher enqueues one kernel on `s` and returns
// the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace k2 {

enum Dt { DT_F32 = 0, DT_BF16 = 1 };

inline size_t dt_size(int dt) { return dt == DT_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------------------------
// GEMM: C[m, n] = sum_k A[m, k] * Bw[n, k]  (A row-major M x K, weights nn.Linear (N, K) layout)
// ---------------------------------------------------------------------------------------------
struct GemmA {
  const void* A;
  int lda;
  int M, K;
};

// q/k/v/gate projection of the block: B rows are the concatenation [to_q; to_k; to_v; to_gate].
// Epilogue: per-head RMSNorm (1 + w) on q and k, then RoPE; v stored transposed per (batch, kv head);
// gate stored as is.
struct QkvgArgs {
  const void* wq; const void* wk; const void* wv; const void* wg;  // (nq, K), (nk, K), (nk, K), (nq, K)
  int nq, nk;                   // nh*hd, nkv*hd
  int hd, L;                    // head dim, tokens per batch row
  void* q; void* k; void* vt; void* g;
  int ldvt;                     // row stride of vt (B, nkv, hd, ldvt)
  const float* wnq; const float* wnk;  // (hd) zero-centred, may be NULL
  const float* rope_cos; const float* rope_sin;  // (L, hd/2) or NULL (no RoPE)
  float eps;
  // optional extra outputs for the backward's recompute (NULL = not written): the raw q and k
  // projections before their norms (float32, (M, nq) and (M, nk)), v row-major (M, nk) in the
  // operand dtype, and k after norm and RoPE transposed like vt (B, nkv, hd, ldvt)
  float* qraw; float* kraw;
  void* vrow; void* kt;
};

// SwiGLU up projection: a = silu(x Wgate^T) * (x Wup^T), a: (M, I).
struct SwigluArgs {
  const void* wgate; const void* wup;
  int I;
  void* a;
  float* gsave; float* usave;  // optional float32 (M, I) copies of x Wgate^T and x Wup^T (NULL = none)
};

// Residual projection: hout[m, n] = hin[m, n] + gate[m / L, n] * (A Bw^T)[m, n]; gate NULL = 1.
struct ResidArgs {
  const void* w;
  int N;
  const float* hin; float* hout;
  const float* gate; int gate_stride;  // gate row b at gate + b * gate_stride
  int L;
};

// Plain projection with bias and optional outputs; output row for input row m is
// (m / rows_per_b) * out_rows_per_b + out_row_off + (m % rows_per_b).
struct PlainArgs {
  const void* w;
  int N;
  const float* bias;            // (N) or NULL
  float* outf; int ldf;         // acc + bias (float), or NULL
  void* outt; int ldt;          // act(acc + bias) in the operand dtype, or NULL
  int act;                      // 0 = identity, 1 = gelu_tanh (applies to outt only)
  int rows_per_b, out_rows_per_b, out_row_off;
};

hipError_t gemm_qkvg(int dt, const GemmA& a, const QkvgArgs& p, hipStream_t s);
hipError_t gemm_swiglu(int dt, const GemmA& a, const SwigluArgs& p, hipStream_t s);
hipError_t gemm_resid(int dt, const GemmA& a, const ResidArgs& p, hipStream_t s);
hipError_t gemm_plain(int dt, const GemmA& a, const PlainArgs& p, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Attention: og[m, h*hd + d] = softmax-attention output * sigmoid(g[m, h*hd + d])
// ---------------------------------------------------------------------------------------------
struct AttnArgs {
  const void* q; const void* k; const void* vt; const void* g;
  void* og;
  const uint8_t* mask;  // (B, T) or NULL
  int B, L, T;
  int nh, nkv, hd;
  int ldvt;
  // Block-causal restriction (NULL = none): query i attends key j only if j <= reach[i]; reach is
  // (L,) and non-decreasing with reach[i] >= i (block_reach builds it from image block ids).
  const int* reach;
  // optional extra outputs for the backward (NULL = not written): the attention output before the
  // gate (M, nh*hd) in the operand dtype, and per (batch, head, query) the log-sum-exp of the
  // scores in base 2 with the scale folded in, log2 sum_j 2^(s_j log2(e) / sqrt(hd)) (+inf for a
  // query with no key)
  void* o_pre;
  float* lse;
};
hipError_t attention(int dt, const AttnArgs& p, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Backward pass (backward.hip)
// ---------------------------------------------------------------------------------------------
struct TransposeArgs {
  const void* src; void* dst;
  int R, C, Rpad;         // source rows and columns; destination row length covered (zeros past R)
  int lds, ldd;           // row strides of source and destination (elements)
  int Z, zdiv;            // batch count; batch z offsets: (z / zdiv) * s0 + (z % zdiv) * s1
  size_t sz0, sz1, dz0, dz1;
};
hipError_t transpose(int dt, const TransposeArgs& p, hipStream_t s);
hipError_t gated_add(const float* h, const float* y, const float* gate, int gate_stride, int L, int M, int H,
                     float* out, hipStream_t s);
struct GatedGradArgs {
  const float* dh; const float* br;   // (B*L, H) float32; br NULL = no partial sums
  const float* gate; int gate_stride; // gate row b, NULL = 1
  void* out;                          // (B*L, H) operand dtype: gate * dh
  float* part;                        // (B * ncb, H) column sums of dh * br per chunk, or NULL
  int B, L, H, RC, ncb;               // chunks of RC rows, ncb = ceil(L / RC) per batch row
};
hipError_t gated_grad(int dt, const GatedGradArgs& p, hipStream_t s);
hipError_t swiglu_bwd(int dt, const float* da, const float* gt, const float* up, int M, int I, void* dgu,
                      hipStream_t s);
struct NormBwdArgs {
  const float* x;      // (B*L, H) the norm's input
  const float* dout;   // (B*L, H) gradient of the modulated output
  const float* dres;   // (B*L, H) added to the input gradient, or NULL
  float* dx;           // (B*L, H) input gradient (may alias dres)
  const float* w;      // (H) zero-centred norm weight or NULL
  const float* scale; int mod_stride;  // modulation scale row b at scale + b * mod_stride, or NULL
  float* pw; float* psc; float* psh;   // (B * ncb, H) partials, each may be NULL
  int B, L, H, RC, ncb;
  float eps;
};
hipError_t norm_bwd(const NormBwdArgs& p, hipStream_t s);
struct GateBwdArgs {
  const float* dog;       // (M, nq) float32 gradient of the gated attention output
  const void* g;          // (M, nq) raw gate projection
  const void* o;          // (M, nq) attention output before the gate
  void* dout;             // (M, nq) gradient of the attention output, operand dtype
  void* dg; int ldg;      // gradient of the raw gate, operand dtype, row stride ldg
  float* delta;           // (B, nh, L)
  int M, L, nh, nq, hd;
};
hipError_t gate_bwd(int dt, const GateBwdArgs& p, hipStream_t s);
struct AttnBwdArgs {
  const void* q; const void* k; const void* v;  // (M, nh*hd), (M, nkv*hd), (M, nkv*hd) row-major
  const void* qt; const void* kt; const void* dot;  // (B, nh, hd, ldt), (B, nkv, hd, ldt), (B, nh, hd, ldt)
  const void* dout;                              // (M, nh*hd) gradient of the attention output
  const float* lse; const float* delta;          // (B, nh, L)
  const uint8_t* mask;                           // (B, T) or NULL
  float* dq; int lddq;                           // (M, .) float32, head h at column h*hd
  float* dk; int lddk;                           // (M, .) float32, kv head at column kvh*hd
  void* dv; int lddv;                            // (M, .) operand dtype
  // (4, M, nkv*hd) float32 scratch: the dK / dV partial sums when the dK/dV pass splits each key
  // block's query tiles over two workgroups (NULL: never split)
  float* dkv_part;
  int B, L, T, nh, nkv, hd, ldt;
};
hipError_t attention_backward(int dt, const AttnBwdArgs& p, hipStream_t s);
struct QkNormBwdArgs {
  const float* dr; int lddr;   // gradient of the rotated, normed heads (float32)
  const float* x; int ldx;     // raw projection (float32)
  const float* rc; const float* rs;  // (L, hd/2) rotation table or NULL
  const float* w;              // (hd) zero-centred norm weight or NULL
  void* dx; int lddx;          // raw projection gradient, operand dtype
  float* part;                 // (blocks, hd) partial sums for the norm weight, or NULL
  int M, L, heads, hd;
  float eps;
};
hipError_t qknorm_bwd(int dt, const QkNormBwdArgs& p, int blocks, hipStream_t s);
hipError_t reduce_rows(const float* part, int G, int nc, int ncols, int ldp, float* out, int ldo, hipStream_t s);
// up to kMaxReduceJobs independent reduce_rows in one launch
struct ReduceJob {
  const float* part; float* out;
  int G, nc, ncols, ldp, ldo;
};
constexpr int kMaxReduceJobs = 12;
struct ReduceJobs {
  ReduceJob job[kMaxReduceJobs];
  int n;
};
hipError_t reduce_rows_multi(const ReduceJobs& jobs, hipStream_t s);

// reach[i] = i for tokens outside every image block (ids[i] < 0), else the last position of the
// contiguous run of equal ids that holds i. One workgroup; ids and reach are (L,) device arrays.
hipError_t block_reach(const int* ids, int L, int* reach, hipStream_t s);

// ---------------------------------------------------------------------------------------------
// Row kernels
// ---------------------------------------------------------------------------------------------
// out[r] = (1 + scale_b) * RMSNorm(in[src_row(r)]; w) + shift_b in the operand dtype, where
// r = b * rows_per_b + i reads input row b * in_rows_per_b + in_row_off + i and
// scale_b = scale + b * mod_stride (NULL = 0), shift_b likewise.
struct ModnormArgs {
  const float* in; void* out;
  int rows, H;
  int rows_per_b, in_rows_per_b, in_row_off;
  const float* w;
  const float* scale; const float* shift; int mod_stride;
  float eps;
};
hipError_t modnorm(int dt, const ModnormArgs& p, hipStream_t s);

// mod[b, c, j] = temb[b * temb_stride + c * chunk_stride + j] + table[c, j] for c < nchunks
// (table may be NULL). chunk_stride = H splits temb into chunks; 0 adds the same vector to every row.
hipError_t modulation(const float* temb, int temb_stride, int chunk_stride, const float* table, float* mod,
                      int B, int nchunks, int H, hipStream_t s);

// cos/sin (L, hd/2) of the 3-axis rotary angles pos[l, a] * theta^(-2i/d_a).
hipError_t rope_table(const float* pos, int L, int a0, int a1, int a2, float theta, float* cos_out,
                      float* sin_out, hipStream_t s);

// Sinusoidal time embedding [cos(1000 t f_k)] ++ [sin(1000 t f_k)] in the operand dtype.
hipError_t time_embed(int dt, const float* t, int B, int dim, void* out, hipStream_t s);

// y[n, d] = sum_l c[l] * x[n, l, d] (float32).
hipError_t layer_compress(const float* x, const float* c, float* y, int rows, int nl, int D, hipStream_t s);

// Element conversion between float32 and the operand dtype.
hipError_t to_f32(int dt, const void* in, float* out, size_t n, hipStream_t s);
hipError_t from_f32(int dt, const float* in, void* out, size_t n, hipStream_t s);

// x_out = x + dsigma * (vc + g (vc - vu)) over n floats (vc alone when vu is NULL); x_out may alias x.
hipError_t cfg_euler(const float* x, float* x_out, const float* vc, const float* vu, size_t n, float g, float dsigma,
                     hipStream_t s);
// out[i] = v for i < n
hipError_t fill_f32(float* out, int n, float v, hipStream_t s);

// Matrix-core rate probe: blocks workgroups of 4 waves, each wave iters x 4 bf16 32x32x16 products
// (blocks * 4 * iters * 4 * 32768 FLOP); writes one float to out[0].
hipError_t mfma_probe(int iters, int blocks, float* out, hipStream_t s);

}  // namespace k2
