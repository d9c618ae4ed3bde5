// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace ssm {

// ---- ternarisation + packing (quant.hip)
hipError_t launch_abs_partials(const float* w, int64_t n, int64_t k, int64_t group, double* part,
                               hipStream_t s);
hipError_t launch_scales(const double* part, int64_t n, int64_t k, int64_t group, const float* scale_in,
                         float* scale, hipStream_t s);
hipError_t launch_pack(const float* w, int64_t n, int64_t k, int64_t group, const float* scale,
                       uint32_t* packed, int64_t* zero_count, hipStream_t s);

// ---- RMSNorm + activation quantisation (norm.hip)
// mode 8: int8 codes q [m, ldo] (zero past k) + absmax [m] (+ optional q2 [m, k]);
// mode 16: bf16 normalised rows xh [m, ldo] (zero past k), and when xh_lo is given the
// remainder xh_lo = bf16(x - xh) so that xh + xh_lo carries about 16 significant bits.
hipError_t launch_norm(const void* x, int x_bf16, int64_t m, int k, int64_t ldx, const float* gain,
                       float eps, int mode, int ldo, int8_t* q, float* absmax, int8_t* q2, bf16_t* xh,
                       bf16_t* xh_lo, hipStream_t s);

// ---- ternary contraction (bitlinear.hip)
struct GemmArgs {
  const void* A;          // int8 (A8) or bf16 (A16) rows [M, lda], zero-padded to Kp columns
  const void* A2;         // A16 only, or null: second bf16 term of each activation (same layout)
  int64_t lda;
  const float* absmax;    // A8: [M]
  const uint32_t* W;      // packed words [N, w_row_words]
  int64_t w_row_words;
  const float* w_scale;   // [1] or [N, K / group]
  int64_t group;          // 0 or a multiple of 64
  int64_t M, N, K, Kp;
  const float* bias;      // [N] or null
  const void* residual;   // [M, ld_res] of the output dtype or null
  int64_t ld_res;
  void* y;
  int64_t ldy;
  int y_bf16;
  int32_t* dbg_acc;       // [M, N] or null (A8)
};
hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t s);

// Row-block A8 BitLinear (norm + int8 codes in LDS + MFMA + epilogue in one kernel), k <= 1024,
// one scale per tensor.
struct RowArgs {
  const void* x;          // rows [M, ldx] (fp32 or bf16)
  int64_t ldx;
  int x_bf16;
  const float* gain;      // RMSNorm gains [K] or null
  float eps;
  int8_t* dbg_xq;         // [M, K] or null
  float* dbg_absmax;      // [M] or null
};
hipError_t launch_bitlinear_rows(const GemmArgs& g, const RowArgs& r, hipStream_t s);
constexpr int64_t kRowsMaxK = 1024;
constexpr int kRowsResN = 512;  // widest residual the row-block kernel stages (more: tiled path)
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t s);

// ---- selective scan (scan.hip: Mamba-1 kind; ssd.hip: SSD kind)
struct ScanArgs {
  int64_t batch, L, H, P, N;
  int act_bf16;
  const void* x; int64_t ld_x;
  const void* delta; int64_t ld_delta;   // pre-activation dt [B, L, H] (unused when fused)
  const float* delta_bias; int softplus;
  const float* A;
  const void* Bm; int64_t ld_B;
  const void* Cm; int64_t ld_C;
  const float* D;
  const float* h0;
  float* h_last;
  void* y; int64_t ld_y;
  // Mamba-1 only: dt computed in the scan from a low-rank input (a BitLinear of k = R)
  const void* dr; int64_t ld_dr; int R;
  const uint32_t* w_dt; int64_t w_dt_row_words;
  const float* s_dt; const float* g_dt; float eps;
  int dt_codes_ready;  // the dt input's int8 codes and factors are already in the workspace
  int32_t* dbg_dt_acc;  // nullable [B L, H]: the in-scan dt projection's int32 sums (stage checks)
  const int8_t* ext_codes; const double* ext_deq;  // nullable: the dt input's codes computed by the caller
  const void* gate; int64_t ld_gate;  // nullable: y is multiplied by SiLU(gate) before it is stored
};
hipError_t launch_scan_m1(const ScanArgs& a, void* ws, hipStream_t s);
// the dt input's int8 codes [M, cw] (cw = 16 ceil(R / 16)) and fp64 factors [M]
hipError_t launch_dt_codes(const void* dr, int bf16, int64_t M, int64_t ld, int R, const float* g, float eps,
                           int8_t* codes, double* deq, hipStream_t s);
size_t scan_m1_workspace(const ScanArgs& a);
// Where the scan keeps the dt input's codes ([M, *cw] int8 at offset 0) and their fp64
// dequantisation factors ([M] at *off_deq) in its workspace.
void scan_m1_code_layout(const ScanArgs& a, int* cw, size_t* off_deq);

// The library's static scratch array on the current device (scan.hip): kStaticScratchBytes,
// 256-byte aligned, shared by every call on that device.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(void** ptr);

// ---- causal depthwise convolution + SiLU (conv.hip)
struct ConvArgs {
  int64_t batch, L, C;
  int K;                        // width, 1 .. kConvMaxK
  int act_bf16;
  const void* x; int64_t ldx;   // [B, L, ldx], channels 0 .. C-1
  const float* w;               // [C, K]
  const float* bias;            // [C] or null
  const float* state_in;        // [B, K-1, C] fp32 or null (zeros before t = 0)
  float* state_out;             // [B, K-1, C] fp32 or null; may equal state_in
  void* out; int64_t ldo;       // [B, L, ldo]
};
constexpr int kConvMaxK = 8;
hipError_t launch_conv_silu(const ConvArgs& a, hipStream_t s);

// ---- full-precision linear layer (dense.hip): y[M, N] = x[M, K] W[N, K]^T (+ residual)
struct DenseArgs {
  int64_t M, N, K;
  int bf16;                      // activations and weights bf16 (else fp32)
  const void* x; int64_t ldx;
  const void* W;                 // [N, K] row-major
  const void* residual; int64_t ld_res;  // nullable; may equal y
  void* y; int64_t ldy;
};
hipError_t launch_dense(const DenseArgs& a, hipStream_t s);
// row-major fp32 C[M, N] = A[M, K] B[K, N], C overwritten
hipError_t sgemm_nn(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                    float* C, int64_t ldc, hipStream_t s);

// ---- straight-through-estimator backward of BitLinear and the QAT update (ste.hip)
struct SteArgs {
  int64_t M, K, N;
  const void* x; int64_t ldx; int x_bf16;
  const float* gain; float eps;
  const uint32_t* W; int64_t w_row_words;
  const float* scale; int64_t group;
  const float* w_latent;          // for the scale gradient
  const float* dy; int64_t ld_dy;  // fp32 [M, N]
  float* dx; int64_t ld_dx;        // fp32 [M, K]
  float* dw;                       // fp32 [N, K] or null
  float* dscale;                   // fp32 [1] or [N, K / group] or null (needs dw and w_latent)
};
size_t ste_workspace(const SteArgs& a);
hipError_t launch_ste_bwd(const SteArgs& a, void* ws, hipStream_t s);
hipError_t launch_sgd(float* w, const float* dw, int64_t n, float lr, hipStream_t s);

// ---- Mamba-1 mixer front (front.hip): x = BitLinear(u; W_in), p = BitLinear(x; W_x) and the
// dt input's int8 codes in one kernel (A8, one scale per tensor)
struct FrontArgs {
  int64_t M;
  const void* u; int act_bf16;
  int Dm, Di, PW, R;
  const uint32_t* w_in; const float* s_in; const float* g_in;
  const uint32_t* w_x; const float* s_x; const float* g_x;
  float eps;
  void* x; void* p;
  const float* g_dt;
  int8_t* codes; int cw; double* deq;
};
bool front_supported(int Dm, int Di, int PW, int R);
// ---- decoding steps of the Mamba-1 kind mixer, ternary projections (decode.hip): one token
// per sequence through nl consecutive layers (the output of layer l is the input of l + 1)
struct DecodeLayer {
  const uint32_t* w_in; const float* s_in; const float* g_in;    // packed [Di, Dm / 16 words]
  const uint32_t* w_x; const float* s_x; const float* g_x;       // packed [PW, Di / 16 words]
  const uint32_t* w_dt; const float* s_dt; const float* g_dt;    // packed [Di, w_dt_row_words]
  const float* dt_bias; const float* A; const float* D;          // [Di], [Di, NS], [Di]
  const uint32_t* w_out; const float* s_out; const float* g_out;  // packed [Dm, Di / 16 words]
  float* state;                                                  // [B, Di, NS], read and written
  int gains;  // bit 0 .. 3: g_in, g_x, g_out, g_dt given
};
constexpr int kDecMaxLayers = 24;  // layers per launch (the kernel argument holds their pointers)
struct DecodeArgs {
  int64_t B;                     // sequences (one token each)
  int Dm, Di, NS, R, PW;         // d_model, d_inner, d_state, dt_rank, x_proj width (R + 2 NS)
  int act_bf16;
  const void* u; void* out; int add_residual;  // [B, Dm] of the activation type
  int64_t w_dt_row_words;
  float eps;
  int nl;                        // layers, 1 .. kDecMaxLayers
  DecodeLayer layer[kDecMaxLayers];
};
bool decode_supported(int Dm, int Di, int NS, int R, int PW);
hipError_t launch_decode_m1(const DecodeArgs& a, hipStream_t s);

hipError_t launch_m1_front(const FrontArgs& f, hipStream_t s);
hipError_t launch_scan_ssd(const ScanArgs& a, void* ws, size_t ws_bytes, hipStream_t s);
size_t scan_ssd_workspace(const ScanArgs& a);

}  // namespace ssm
