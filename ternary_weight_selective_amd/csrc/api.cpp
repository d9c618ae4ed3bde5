// C ABI entry points: host-side validation, workspace carving and launch sequencing.
// Nothing here touches device memory except through kernel launches on the caller's stream.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.hpp"
#include "mixer_bwd.hpp"
#include "scan_bwd.hpp"
#include "ssm_ternary.h"

using namespace ssm;

namespace {

thread_local std::string g_err;

ssm_status fail(ssm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ssm_status dev(hipError_t e, const char* what) {
  if (e == hipSuccess) return SSM_OK;
  return fail(SSM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool act_dtype_ok(int32_t t) { return t == SSM_F32 || t == SSM_BF16; }
size_t act_size(int32_t t) { return t == SSM_BF16 ? 2 : 4; }
constexpr int64_t kMaxK = 4096;

// ------------------------------------------------------------------ BitLinear

struct BLPlan {
  int64_t Kp = 0;
  bool norm = false;
  bool rows = false;  // row-block kernel (A8, one scale per tensor, k <= 1024)
  size_t off_am = 0, total = 0;
};

// The row-block kernel keeps a projection's packed weights in registers when each consumer
// wave's run of 16-column tiles fits one round (k <= 64 KPL with KPL a power of two, up to
// min(32 / KPL, 8) tiles per wave, four consumer waves); wider projections reload their weights
// for every 16-row block.  From kRowsBigM rows on, when the large-tile contraction has at least
// one 256 x 128 tile per compute unit, the norm kernel + that contraction is faster (TernarySSM
// shape, 16384 tokens, bf16: in_proj 512 -> 1024 52.6 -> 34 us, out_proj 1024 -> 512 50.5 ->
// 45 us).  Both paths give the same bits (same codes, int32 sums and fp64 epilogue).
constexpr int64_t kRowsBigM = 2048;
bool rows_one_round(int64_t k, int64_t n) {
  int64_t kpl = 1;
  while (64 * kpl < k) kpl *= 2;
  const int64_t tpr = 32 / kpl < 8 ? 32 / kpl : 8;
  return cdiv(cdiv(n, 16), 4) <= tpr;
}

ssm_status bl_plan(const ssm_bitlinear_args* a, BLPlan* p) {
  if (!a) return fail(SSM_ERR_NULL, "bitlinear: args is NULL");
  if (a->act_bits != 8 && a->act_bits != 16) return fail(SSM_ERR_UNSUPPORTED, "bitlinear: act_bits must be 8 or 16");
  if (a->x_dtype != SSM_F32 && a->x_dtype != SSM_BF16 && a->x_dtype != SSM_I8)
    return fail(SSM_ERR_DTYPE, "bitlinear: x_dtype %d", a->x_dtype);
  if (a->x_dtype == SSM_I8 && a->act_bits != 8) return fail(SSM_ERR_DTYPE, "bitlinear: int8 input needs act_bits 8");
  if (!act_dtype_ok(a->y_dtype)) return fail(SSM_ERR_DTYPE, "bitlinear: y_dtype %d", a->y_dtype);
  if (a->m < 0) return fail(SSM_ERR_SHAPE, "bitlinear: m = %lld", (long long)a->m);
  if (a->k < 1 || a->k > kMaxK) return fail(SSM_ERR_SHAPE, "bitlinear: k = %lld not in [1, %lld]", (long long)a->k, (long long)kMaxK);
  if (a->n_out < 1 || a->n_out > (1LL << 24)) return fail(SSM_ERR_SHAPE, "bitlinear: n_out = %lld", (long long)a->n_out);
  if (a->ldx < a->k) return fail(SSM_ERR_SHAPE, "bitlinear: ldx %lld < k %lld", (long long)a->ldx, (long long)a->k);
  if (a->ldy < a->n_out) return fail(SSM_ERR_SHAPE, "bitlinear: ldy %lld < n_out %lld", (long long)a->ldy, (long long)a->n_out);
  if (a->residual && a->ld_res < a->n_out) return fail(SSM_ERR_SHAPE, "bitlinear: ld_res < n_out");
  if (a->group_size < 0 || (a->group_size > 0 && (a->group_size % 64 != 0 || a->k % a->group_size != 0)))
    return fail(SSM_ERR_SHAPE, "bitlinear: group_size %lld must be 0 or a multiple of 64 dividing k", (long long)a->group_size);
  if (!a->w_packed || !a->w_scale) return fail(SSM_ERR_NULL, "bitlinear: w_packed / w_scale is NULL");
  if (!aligned(a->w_packed, 4)) return fail(SSM_ERR_ALIGN, "bitlinear: w_packed must be 4-byte aligned");
  if (a->m > 0 && (!a->x || !a->y)) return fail(SSM_ERR_NULL, "bitlinear: x / y is NULL");
  if (a->act_bits == 16 && (a->dbg_xq || a->dbg_absmax || a->dbg_acc))
    return fail(SSM_ERR_UNSUPPORTED, "bitlinear: stage outputs exist for act_bits 8 only");
  p->Kp = round_up(a->k, 64);
  p->norm = a->x_dtype != SSM_I8;
  if (!p->norm) {
    if (!a->x_absmax && a->m > 0) return fail(SSM_ERR_NULL, "bitlinear: x_absmax is required for int8 input");
    if (a->k % 64 != 0 || a->ldx % 16 != 0 || !aligned(a->x, 16))
      return fail(SSM_ERR_UNSUPPORTED, "bitlinear: int8 input needs k %% 64 == 0, ldx %% 16 == 0, 16-byte alignment");
    p->total = 0;
    return SSM_OK;
  }
  if (a->act_bits == 8 && a->group_size == 0 && a->k <= kRowsMaxK && (!a->residual || a->n_out <= kRowsResN) &&
      (a->m < kRowsBigM || rows_one_round(a->k, a->n_out) || cdiv(a->m, 256) * cdiv(a->n_out, 128) < 256)) {
    p->rows = true;
    p->total = 0;
    return SSM_OK;
  }
  // A8: int8 codes; A16: bf16 rows, two terms (hi, lo) when the output is fp32
  const size_t elt = a->act_bits == 8 ? 1 : (a->y_dtype == SSM_F32 ? 4 : 2);
  p->off_am = align_up((size_t)a->m * p->Kp * elt);
  p->total = a->act_bits == 8 ? align_up(p->off_am + (size_t)a->m * 4) : p->off_am;
  return SSM_OK;
}

// Runs a planned BitLinear with its workspace.
ssm_status bl_run(const ssm_bitlinear_args* a, const BLPlan& p, void* ws, hipStream_t s) {
  if (a->m == 0) return SSM_OK;
  GemmArgs g{};
  g.W = (const uint32_t*)a->w_packed;
  g.w_row_words = cdiv(a->k, 16);
  g.w_scale = a->w_scale;
  g.group = a->group_size;
  g.M = a->m;
  g.N = a->n_out;
  g.K = a->k;
  g.Kp = p.Kp;
  g.bias = a->bias;
  g.residual = a->residual;
  g.ld_res = a->ld_res;
  g.y = a->y;
  g.ldy = a->ldy;
  g.y_bf16 = a->y_dtype == SSM_BF16;
  g.dbg_acc = a->dbg_acc;
  if (!p.norm) {
    g.A = a->x;
    g.lda = a->ldx;
    g.absmax = a->x_absmax;
    return dev(launch_gemm_i8(g, s), "bitlinear gemm");
  }
  const int xb = a->x_dtype == SSM_BF16;
  if (p.rows) {  // row-block kernel: norm, codes, contraction and epilogue in one launch
    RowArgs r{};
    r.x = a->x; r.ldx = a->ldx; r.x_bf16 = xb;
    r.gain = a->norm_weight; r.eps = a->norm_eps;
    r.dbg_xq = a->dbg_xq; r.dbg_absmax = a->dbg_absmax;
    return dev(launch_bitlinear_rows(g, r, s), "bitlinear rows");
  }
  if (a->act_bits == 8) {
    int8_t* q = (int8_t*)ws;
    float* am = a->dbg_absmax ? a->dbg_absmax : (float*)((char*)ws + p.off_am);
    ssm_status st = dev(launch_norm(a->x, xb, a->m, (int)a->k, a->ldx, a->norm_weight, a->norm_eps, 8, (int)p.Kp, q,
                                    am, a->dbg_xq, nullptr, nullptr, s),
                        "bitlinear norm");
    if (st != SSM_OK) return st;
    g.A = q;
    g.lda = p.Kp;
    g.absmax = am;
    return dev(launch_gemm_i8(g, s), "bitlinear gemm");
  }
  bf16_t* xh = (bf16_t*)ws;
  bf16_t* xh_lo = a->y_dtype == SSM_F32 ? xh + (size_t)a->m * p.Kp : nullptr;
  ssm_status st = dev(launch_norm(a->x, xb, a->m, (int)a->k, a->ldx, a->norm_weight, a->norm_eps, 16, (int)p.Kp,
                                  nullptr, nullptr, nullptr, xh, xh_lo, s),
                      "bitlinear norm");
  if (st != SSM_OK) return st;
  g.A = xh;
  g.A2 = xh_lo;
  g.lda = p.Kp;
  return dev(launch_gemm_bf16(g, s), "bitlinear gemm");
}

// ------------------------------------------------------------------ scan

ssm_status scan_check(const ssm_scan_args* a) {
  if (!a) return fail(SSM_ERR_NULL, "scan: args is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(SSM_ERR_SHAPE, "scan: negative batch / seqlen");
  if (a->nheads < 1 || a->headdim < 1 || a->d_state < 1) return fail(SSM_ERR_SHAPE, "scan: nheads, headdim, d_state must be >= 1");
  if (!act_dtype_ok(a->act_dtype)) return fail(SSM_ERR_DTYPE, "scan: act_dtype %d", a->act_dtype);
  if (a->a_per_state == 1) {
    if (a->headdim != 1) return fail(SSM_ERR_UNSUPPORTED, "scan: a_per_state = 1 needs headdim = 1");
    const int64_t n = a->d_state;
    if (n != 4 && n != 8 && n != 16 && n != 32 && n != 64) return fail(SSM_ERR_UNSUPPORTED, "scan: d_state %lld (Mamba-1 kind: 4, 8, 16, 32, 64)", (long long)n);
  } else if (a->a_per_state == 0) {
    const int64_t n = a->d_state;
    if (n != 16 && n != 32 && n != 64 && n != 128) return fail(SSM_ERR_UNSUPPORTED, "scan: d_state %lld (SSD kind: 16, 32, 64, 128)", (long long)n);
    if (a->headdim > 256) return fail(SSM_ERR_UNSUPPORTED, "scan: headdim %lld > 256", (long long)a->headdim);
  } else {
    return fail(SSM_ERR_SHAPE, "scan: a_per_state must be 0 or 1");
  }
  const int64_t HP = a->nheads * a->headdim;
  const bool proj = a->dt_in != nullptr;
  if (a->ld_x < HP || a->ld_y < HP || a->ld_B < a->d_state || a->ld_C < a->d_state || (!proj && a->ld_delta < a->nheads))
    return fail(SSM_ERR_SHAPE, "scan: a row stride is smaller than its row");
  if (proj) {
    if (a->a_per_state != 1) return fail(SSM_ERR_UNSUPPORTED, "scan: the dt projection exists for the Mamba-1 kind only");
    if (a->dt_rank < 1 || a->dt_rank > 64) return fail(SSM_ERR_UNSUPPORTED, "scan: dt_rank must be in [1, 64]");
    if (a->ld_dt_in < a->dt_rank) return fail(SSM_ERR_SHAPE, "scan: ld_dt_in < dt_rank");
    if (!a->w_dt || !a->s_dt) return fail(SSM_ERR_NULL, "scan: w_dt and s_dt are required with dt_in");
    if (!aligned(a->w_dt, 4)) return fail(SSM_ERR_ALIGN, "scan: w_dt must be 4-byte aligned");
  }
  if (a->batch * a->seqlen > 0 && (!a->x || (!proj && !a->delta) || !a->A || !a->Bm || !a->Cm || !a->y))
    return fail(SSM_ERR_NULL, "scan: x, delta (or dt_in), A, Bm, Cm and y are required");
  if (a->gate && a->ld_gate < HP) return fail(SSM_ERR_SHAPE, "scan: ld_gate < nheads * headdim");
  if (a->dt_codes && (!proj || !a->dt_deq))
    return fail(SSM_ERR_NULL, "scan: dt_codes needs dt_in (for dt_rank) and dt_deq");
  if (a->dt_codes && !aligned(a->dt_codes, 16)) return fail(SSM_ERR_ALIGN, "scan: dt_codes must be 16-byte aligned");
  if (a->a_per_state == 1) {  // the Mamba-1 kind kernel addresses one sequence of a tensor with 32-bit byte offsets
    int64_t ld = a->ld_x > a->ld_y ? a->ld_x : a->ld_y;
    if (a->ld_B > ld) ld = a->ld_B;
    if (a->ld_C > ld) ld = a->ld_C;
    if (!proj && a->ld_delta > ld) ld = a->ld_delta;
    if (a->gate && a->ld_gate > ld) ld = a->ld_gate;
    if (ld < 64) ld = 64;  // the dt codes: <= 64 bytes per token
    if (a->seqlen * ld * (int64_t)act_size(a->act_dtype) >= (int64_t(1) << 31))
      return fail(SSM_ERR_UNSUPPORTED, "scan: one sequence spans 2 GiB or more of a tensor");
  }
  return SSM_OK;
}

ScanArgs to_scan(const ssm_scan_args* a) {
  ScanArgs s{};
  s.batch = a->batch;
  s.L = a->seqlen;
  s.H = a->nheads;
  s.P = a->headdim;
  s.N = a->d_state;
  s.act_bf16 = a->act_dtype == SSM_BF16;
  s.x = a->x; s.ld_x = a->ld_x;
  s.delta = a->delta; s.ld_delta = a->ld_delta;
  s.delta_bias = a->delta_bias; s.softplus = a->delta_softplus;
  s.A = a->A;
  s.Bm = a->Bm; s.ld_B = a->ld_B;
  s.Cm = a->Cm; s.ld_C = a->ld_C;
  s.D = a->D; s.h0 = a->h0; s.h_last = a->h_last;
  s.y = a->y; s.ld_y = a->ld_y;
  s.gate = a->gate; s.ld_gate = a->ld_gate;
  if (a->dt_in) {
    s.dr = a->dt_in; s.ld_dr = a->ld_dt_in; s.R = (int)a->dt_rank;
    s.w_dt = (const uint32_t*)a->w_dt; s.w_dt_row_words = cdiv(a->dt_rank, 16);
    s.s_dt = a->s_dt; s.g_dt = a->g_dt; s.eps = a->dt_eps;
    s.ext_codes = a->dt_codes; s.ext_deq = a->dt_deq;
  }
  return s;
}

// ------------------------------------------------------------------ mixer

struct MixPlan {
  int64_t M = 0, Kp = 0, PW = 0, VW = 0;
  int64_t XW = 0;   // Mamba-1: in_proj width (d_inner, or 2 d_inner with the gate branch)
  int64_t VW0 = 0;  // SSD: [x | B | C | dt] width; VW adds the gate branch
  int64_t Cc = 0;   // channels through the convolution of the gated block
  size_t off_am = 0, off_x = 0, off_xc = 0, off_p = 0, off_dl = 0, off_y = 0, off_scan = 0, total = 0;
};

ssm_status mix_plan(const ssm_mixer_config* c, int64_t batch, int64_t seqlen, MixPlan* p) {
  if (!c) return fail(SSM_ERR_NULL, "mixer: config is NULL");
  if (batch < 0 || seqlen < 0) return fail(SSM_ERR_SHAPE, "mixer: negative batch / seqlen");
  if (!act_dtype_ok(c->act_dtype)) return fail(SSM_ERR_DTYPE, "mixer: act_dtype %d", c->act_dtype);
  if (c->d_model < 1 || c->d_model > kMaxK || c->d_inner < 1 || c->d_inner > kMaxK)
    return fail(SSM_ERR_SHAPE, "mixer: d_model and d_inner must be in [1, %lld]", (long long)kMaxK);
  if (c->act_bits != 8 && c->act_bits != 16) return fail(SSM_ERR_UNSUPPORTED, "mixer: act_bits must be 8 or 16");
  if (c->group_size < 0 || (c->group_size > 0 && (c->group_size % 64 || c->d_model % c->group_size || c->d_inner % c->group_size)))
    return fail(SSM_ERR_SHAPE, "mixer: group_size must be 0 or a multiple of 64 dividing d_model and d_inner");
  if (c->gated != 0 && c->gated != 1) return fail(SSM_ERR_SHAPE, "mixer: gated must be 0 or 1");
  if (c->gated ? (c->d_conv < 1 || c->d_conv > kConvMaxK) : c->d_conv != 0)
    return fail(SSM_ERR_SHAPE, "mixer: d_conv %d (1 .. %d with gated = 1, else 0)", (int)c->d_conv, kConvMaxK);
  if (c->fp_proj < 0 || c->fp_proj > 2) return fail(SSM_ERR_SHAPE, "mixer: fp_proj must be 0, 1 or 2");
  p->M = batch * seqlen;
  p->Kp = round_up(c->d_model > c->d_inner ? c->d_model : c->d_inner, 64);
  const size_t as = act_size(c->act_dtype);
  size_t off = 0;
  const size_t qbytes = (size_t)p->M * p->Kp * (c->act_bits == 8 ? 1 : (c->act_dtype == SSM_F32 ? 4 : 2));
  off = align_up(qbytes);
  p->off_am = off;
  off = align_up(off + (size_t)p->M * 4);
  if (c->kind == SSM_MIXER_MAMBA1) {
    if (c->act_bits != 8 || c->group_size != 0) return fail(SSM_ERR_UNSUPPORTED, "mixer: Mamba-1 kind needs act_bits 8 and group_size 0");
    if (c->dt_rank < 1 || c->dt_rank > 64) return fail(SSM_ERR_UNSUPPORTED, "mixer: dt_rank must be in [1, 64]");
    const int64_t n = c->d_state;
    if (n != 4 && n != 8 && n != 16 && n != 32 && n != 64) return fail(SSM_ERR_UNSUPPORTED, "mixer: d_state %lld", (long long)n);
    p->PW = c->dt_rank + 2 * c->d_state;
    p->XW = c->gated ? 2 * c->d_inner : c->d_inner;
    p->Cc = c->d_inner;
    p->off_x = off; off = align_up(off + (size_t)p->M * p->XW * as);
    if (c->gated) { p->off_xc = off; off = align_up(off + (size_t)p->M * c->d_inner * as); }
    p->off_p = off; off = align_up(off + (size_t)p->M * p->PW * as);
    if (c->fp_proj == 2) { p->off_dl = off; off = align_up(off + (size_t)p->M * c->d_inner * as); }  // stored dt
    p->off_y = off; off = align_up(off + (size_t)p->M * c->d_inner * as);
    p->off_scan = off;
    const int64_t wmax = p->XW > p->PW ? p->XW : p->PW;  // widest row the scan reads (32-bit offsets per sequence)
    if (seqlen * (wmax > 64 ? wmax : 64) * (int64_t)as >= (int64_t(1) << 31))
      return fail(SSM_ERR_UNSUPPORTED, "mixer: one sequence spans 2 GiB or more of an activation tensor");
  } else if (c->kind == SSM_MIXER_SSD) {
    if (c->nheads < 1 || c->headdim < 1 || c->nheads * c->headdim != c->d_inner)
      return fail(SSM_ERR_SHAPE, "mixer: nheads * headdim must equal d_inner");
    const int64_t n = c->d_state;
    if (n != 16 && n != 32 && n != 64 && n != 128) return fail(SSM_ERR_UNSUPPORTED, "mixer: d_state %lld", (long long)n);
    p->VW0 = c->d_inner + 2 * c->d_state + c->nheads;
    p->VW = c->gated ? p->VW0 + c->d_inner : p->VW0;
    p->Cc = c->d_inner + 2 * c->d_state;
    p->off_p = off; off = align_up(off + (size_t)p->M * p->VW * as);
    if (c->gated) { p->off_xc = off; off = align_up(off + (size_t)p->M * p->Cc * as); }
    p->off_y = off; off = align_up(off + (size_t)p->M * c->d_inner * as);
    p->off_scan = off;
  } else {
    return fail(SSM_ERR_UNSUPPORTED, "mixer: kind %d", c->kind);
  }
  p->total = off;
  return SSM_OK;
}

ssm_status ste_check(const ssm_bitlinear_bwd_args* a, SteArgs* o) {
  if (!a) return fail(SSM_ERR_NULL, "bitlinear bwd: args is NULL");
  if (a->x_dtype != SSM_F32 && a->x_dtype != SSM_BF16) return fail(SSM_ERR_DTYPE, "bitlinear bwd: x_dtype %d", a->x_dtype);
  if (a->m < 0 || a->k < 1 || a->k > kMaxK || a->n_out < 1 || a->n_out > 0x7fffffff || a->m > 0x7fffffff)
    return fail(SSM_ERR_SHAPE, "bitlinear bwd: m >= 0, 1 <= k <= %lld, n_out >= 1", (long long)kMaxK);
  if (a->ldx < a->k || a->ld_dy < a->n_out || a->ld_dx < a->k)
    return fail(SSM_ERR_SHAPE, "bitlinear bwd: a row stride is smaller than its row");
  // the kernels address a tile of up to 32 rows with 32-bit offsets from its first row
  const int64_t kMaxLd = ((1ll << 31) - 1) / 33;
  if (a->ldx > kMaxLd || a->ld_dy > kMaxLd || a->ld_dx > kMaxLd)
    return fail(SSM_ERR_UNSUPPORTED, "bitlinear bwd: row strides above %lld elements are not supported",
                (long long)kMaxLd);
  if (a->group_size < 0 || (a->group_size > 0 && (a->group_size % 64 != 0 || a->k % a->group_size != 0)))
    return fail(SSM_ERR_SHAPE, "bitlinear bwd: group_size must be 0 or a multiple of 64 dividing k");
  if (!a->w_packed || !a->w_scale) return fail(SSM_ERR_NULL, "bitlinear bwd: w_packed / w_scale is NULL");
  if (!aligned(a->w_packed, 4)) return fail(SSM_ERR_ALIGN, "bitlinear bwd: w_packed must be 4-byte aligned");
  if (a->m > 0 && (!a->x || !a->dy || !a->dx)) return fail(SSM_ERR_NULL, "bitlinear bwd: x, dy and dx are required");
  if (a->d_scale && (!a->dw || !a->w_latent))
    return fail(SSM_ERR_NULL, "bitlinear bwd: d_scale needs dw and w_latent");
  SteArgs& s = *o;
  s = SteArgs{};
  s.M = a->m; s.K = a->k; s.N = a->n_out;
  s.x = a->x; s.ldx = a->ldx; s.x_bf16 = a->x_dtype == SSM_BF16;
  s.gain = a->norm_weight; s.eps = a->norm_eps;
  s.W = (const uint32_t*)a->w_packed; s.w_row_words = cdiv(a->k, 16);
  s.scale = a->w_scale; s.group = a->group_size;
  s.w_latent = a->w_latent;
  s.dy = a->dy; s.ld_dy = a->ld_dy;
  s.dx = a->dx; s.ld_dx = a->ld_dx;
  s.dw = a->dw; s.dscale = a->d_scale;
  return SSM_OK;
}

ssm_status scan_bwd_check(const ssm_scan_bwd_args* a, ScanBwdArgs* o) {
  if (!a) return fail(SSM_ERR_NULL, "scan bwd: args is NULL");
  if (!act_dtype_ok(a->act_dtype)) return fail(SSM_ERR_DTYPE, "scan bwd: act_dtype %d", a->act_dtype);
  if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1) return fail(SSM_ERR_SHAPE, "scan bwd: batch, seqlen >= 0, nheads >= 1");
  const int64_t n = a->d_state;
  if (n != 4 && n != 8 && n != 16 && n != 32 && n != 64) return fail(SSM_ERR_UNSUPPORTED, "scan bwd: d_state %lld", (long long)n);
  if (a->batch > 65535) return fail(SSM_ERR_UNSUPPORTED, "scan bwd: batch above 65535");
  if ((a->seqlen + 256 / n - 1) / (256 / n) > 65535)  // time chunks of 256 / d_state steps
    return fail(SSM_ERR_UNSUPPORTED, "scan bwd: seqlen above %lld for d_state %lld", (long long)(65535 * (256 / n)),
                (long long)n);
  if (a->ld_x < a->nheads || a->ld_delta < a->nheads || a->ld_B < n || a->ld_C < n || a->ld_dy < a->nheads)
    return fail(SSM_ERR_SHAPE, "scan bwd: a row stride is smaller than its row");
  if (a->batch * a->seqlen > 0 && (!a->x || !a->delta || !a->A || !a->Bm || !a->Cm || !a->dy || !a->dx ||
                                   !a->ddelta || !a->dA || !a->dB || !a->dC))
    return fail(SSM_ERR_NULL, "scan bwd: x, delta, A, Bm, Cm, dy, dx, ddelta, dA, dB and dC are required");
  if (!aligned(a->A, 4)) return fail(SSM_ERR_ALIGN, "scan bwd: A must be 4-byte aligned");
  ScanBwdArgs& s = *o;
  s = ScanBwdArgs{};
  s.batch = a->batch; s.L = a->seqlen; s.H = a->nheads; s.N = n;
  s.act_bf16 = a->act_dtype == SSM_BF16; s.softplus = a->delta_softplus;
  s.x = a->x; s.ld_x = a->ld_x; s.delta = a->delta; s.ld_delta = a->ld_delta;
  s.delta_bias = a->delta_bias; s.A = a->A;
  s.Bm = a->Bm; s.ld_B = a->ld_B; s.Cm = a->Cm; s.ld_C = a->ld_C;
  s.D = a->D; s.h0 = a->h0; s.dy = a->dy; s.ld_dy = a->ld_dy;
  s.dx = a->dx; s.ddelta = a->ddelta; s.dA = a->dA; s.dB = a->dB; s.dC = a->dC;
  s.dD = a->dD; s.dbias = a->dbias; s.dh0 = a->dh0;
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(int s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid size or stride";
    case SSM_ERR_DTYPE: return "unsupported dtype";
    case SSM_ERR_ALIGN: return "misaligned pointer or stride";
    case SSM_ERR_WORKSPACE: return "workspace missing or too small";
    case SSM_ERR_UNSUPPORTED: return "unsupported configuration";
    case SSM_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ssm_last_error(void) { return g_err.c_str(); }

int64_t ssm_packed_row_bytes(int64_t k) { return k <= 0 ? 0 : 4 * ((k + 15) / 16); }

size_t ssm_ternary_quantize_workspace_bytes(int64_t n_out, int64_t k, int64_t group_size, const float* scale_in) {
  if (scale_in || n_out < 1 || k < 1 || group_size < 0 || (group_size > 0 && k % group_size)) return 0;
  return (size_t)n_out * (group_size ? k / group_size : 1) * sizeof(double);
}

ssm_status ssm_ternary_quantize_weights(const float* w, int64_t n, int64_t k, int64_t group, const float* scale_in,
                                        uint8_t* packed, float* scale, int64_t* zero_count, void* ws, size_t wsb,
                                        hipStream_t stream) {
  g_err.clear();
  if (!w || !packed || !scale) return fail(SSM_ERR_NULL, "quantize: w_latent, w_packed and w_scale are required");
  if (n < 1 || k < 1) return fail(SSM_ERR_SHAPE, "quantize: n_out = %lld, k = %lld", (long long)n, (long long)k);
  if (group < 0 || (group > 0 && k % group)) return fail(SSM_ERR_SHAPE, "quantize: group_size %lld does not divide k", (long long)group);
  if (!aligned(packed, 4)) return fail(SSM_ERR_ALIGN, "quantize: w_packed must be 4-byte aligned");
  const size_t need = ssm_ternary_quantize_workspace_bytes(n, k, group, scale_in);
  if (need && (!ws || wsb < need)) return fail(SSM_ERR_WORKSPACE, "quantize: workspace needs %zu bytes", need);
  if (need && !aligned(ws, 8)) return fail(SSM_ERR_ALIGN, "quantize: workspace must be 8-byte aligned");
  ssm_status st;
  if (!scale_in) {
    st = dev(launch_abs_partials(w, n, k, group, (double*)ws, stream), "quantize partials");
    if (st != SSM_OK) return st;
  }
  st = dev(launch_scales((const double*)ws, n, k, group, scale_in, scale, stream), "quantize scales");
  if (st != SSM_OK) return st;
  return dev(launch_pack(w, n, k, group, scale, (uint32_t*)packed, zero_count, stream), "quantize pack");
}

size_t ssm_bitlinear_workspace_bytes(const ssm_bitlinear_args* a) {
  BLPlan p;
  std::string keep = g_err;
  const ssm_status st = bl_plan(a, &p);
  g_err = keep;
  return st == SSM_OK ? p.total : 0;
}

ssm_status ssm_bitlinear_fwd(const ssm_bitlinear_args* a, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  BLPlan p;
  ssm_status st = bl_plan(a, &p);
  if (st != SSM_OK) return st;
  if (p.total && (!ws || wsb < p.total)) return fail(SSM_ERR_WORKSPACE, "bitlinear: workspace needs %zu bytes", p.total);
  if (p.total && !aligned(ws, 16)) return fail(SSM_ERR_ALIGN, "bitlinear: workspace must be 16-byte aligned");
  return bl_run(a, p, ws, stream);
}

size_t ssm_selective_scan_workspace_bytes(const ssm_scan_args* a) {
  std::string keep = g_err;
  const ssm_status st = scan_check(a);
  g_err = keep;
  if (st != SSM_OK) return 0;
  return a->a_per_state ? scan_m1_workspace(to_scan(a)) : scan_ssd_workspace(to_scan(a));
}

ssm_status ssm_selective_scan_fwd(const ssm_scan_args* a, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  ssm_status st = scan_check(a);
  if (st != SSM_OK) return st;
  const ScanArgs s = to_scan(a);
  const size_t need = a->a_per_state ? scan_m1_workspace(s) : scan_ssd_workspace(s);
  if (need && (!ws || wsb < need)) return fail(SSM_ERR_WORKSPACE, "scan: workspace needs %zu bytes", need);
  if (need && !aligned(ws, 16)) return fail(SSM_ERR_ALIGN, "scan: workspace must be 16-byte aligned");
  if (a->a_per_state) return dev(launch_scan_m1(s, ws, stream), "scan");
  return dev(launch_scan_ssd(s, ws, wsb, stream), "scan");
}

ssm_status ssm_selective_scan_fwd_noalloc(const ssm_scan_args* a, hipStream_t stream) {
  g_err.clear();
  ssm_status st = scan_check(a);
  if (st != SSM_OK) return st;
  const ScanArgs s = to_scan(a);
  const size_t need = a->a_per_state ? scan_m1_workspace(s) : scan_ssd_workspace(s);
  static_assert(kStaticScratchBytes == SSM_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
  if (need > kStaticScratchBytes)
    return fail(SSM_ERR_UNSUPPORTED, "scan noalloc: needs %zu bytes of scratch, more than the %zu the library holds",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need) {
    st = dev(static_scratch(&ws), "scan noalloc scratch");
    if (st != SSM_OK) return st;
  }
  if (a->a_per_state) return dev(launch_scan_m1(s, ws, stream), "scan noalloc");
  return dev(launch_scan_ssd(s, ws, kStaticScratchBytes, stream), "scan noalloc");
}

size_t ssm_mixer_workspace_bytes(const ssm_mixer_config* c, int64_t batch, int64_t seqlen) {
  std::string keep = g_err;
  MixPlan p;
  const ssm_status st = mix_plan(c, batch, seqlen, &p);
  g_err = keep;
  if (st != SSM_OK) return 0;
  ScanArgs s{};
  s.batch = batch; s.L = seqlen; s.N = c->d_state;
  if (c->kind == SSM_MIXER_SSD) {
    s.H = c->nheads; s.P = c->headdim;
    return p.total + align_up(scan_ssd_workspace(s));
  }
  s.H = c->d_inner; s.P = 1;
  s.R = c->fp_proj == 2 ? 0 : (int)c->dt_rank;  // a ternary dt_proj runs inside the scan: its input's codes
  return p.total + align_up(scan_m1_workspace(s));
}

int32_t ssm_mixer_fuses_front(const ssm_mixer_config* c) {
  std::string keep = g_err;
  MixPlan p;
  const ssm_status st = mix_plan(c, 1, 1, &p);
  g_err = keep;
  if (st != SSM_OK || c->kind != SSM_MIXER_MAMBA1 || c->gated || c->fp_proj) return 0;
  return front_supported((int)c->d_model, (int)c->d_inner, (int)p.PW, (int)c->dt_rank) ? 1 : 0;
}

namespace {
// The decode kernel's conditions for one layer: Mamba-1 kind, ternary projections with
// per-tensor scales and int8 activations, no gate, sizes it is built for, 16-byte aligned
// packed weights, gains, A and state.
bool dec_layer_ok(const ssm_mixer_config* c, const ssm_mixer_weights* w, const float* state, int64_t batch,
                  int64_t pw) {
  return c->kind == SSM_MIXER_MAMBA1 && w && state && !c->gated && !c->fp_proj && c->act_bits == 8 &&
         c->group_size == 0 && batch <= 1024 && w->w_in && w->w_x && w->w_dt && w->w_out && w->s_in && w->s_x &&
         w->s_dt && w->s_out && w->A && aligned(w->w_in, 16) && aligned(w->w_x, 16) && aligned(w->w_out, 16) &&
         aligned(w->A, 16) && aligned(state, 16) && aligned(w->g_in, 16) && aligned(w->g_x, 16) &&
         aligned(w->g_out, 16) && aligned(w->g_dt, 16) &&
         decode_supported((int)c->d_model, (int)c->d_inner, (int)c->d_state, (int)c->dt_rank, (int)pw);
}
DecodeArgs dec_args(const ssm_mixer_config* c, int64_t batch, int64_t pw, const void* u, void* out,
                    int32_t add_residual) {
  DecodeArgs da{};
  da.B = batch; da.Dm = (int)c->d_model; da.Di = (int)c->d_inner; da.NS = (int)c->d_state;
  da.R = (int)c->dt_rank; da.PW = (int)pw; da.act_bf16 = c->act_dtype == SSM_BF16;
  da.u = u; da.out = out; da.add_residual = add_residual ? 1 : 0;
  da.w_dt_row_words = cdiv(c->dt_rank, 16);
  da.eps = c->norm_eps;
  return da;
}
void dec_layer(DecodeLayer& L, const ssm_mixer_weights* w, float* state) {
  L.w_in = (const uint32_t*)w->w_in; L.s_in = w->s_in; L.g_in = w->g_in;
  L.w_x = (const uint32_t*)w->w_x; L.s_x = w->s_x; L.g_x = w->g_x;
  L.w_dt = (const uint32_t*)w->w_dt; L.s_dt = w->s_dt; L.g_dt = w->g_dt;
  L.dt_bias = w->dt_bias; L.A = w->A; L.D = w->D;
  L.w_out = (const uint32_t*)w->w_out; L.s_out = w->s_out; L.g_out = w->g_out;
  L.state = state;
  L.gains = (w->g_in ? 1 : 0) | (w->g_x ? 2 : 0) | (w->g_out ? 4 : 0) | (w->g_dt ? 8 : 0);
}

// One mixer layer; state (nullable): the scan's initial state, overwritten with its final state
// (used for one token per sequence only, where no time chunks are formed).
ssm_status mixer_run(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                     int64_t batch, int64_t seqlen, int32_t add_residual, void* ws, size_t wsb, hipStream_t stream,
                     float* state, float* conv_state, const ssm_mixer_stages* dbg);
}  // namespace

ssm_status ssm_mixer_fwd(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                         int64_t batch, int64_t seqlen, int32_t add_residual, void* ws, size_t wsb,
                         hipStream_t stream) {
  g_err.clear();
  return mixer_run(c, w, u, out, batch, seqlen, add_residual, ws, wsb, stream, nullptr, nullptr, nullptr);
}

ssm_status ssm_mixer_fwd_stages(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                                int64_t batch, int64_t seqlen, int32_t add_residual, void* ws, size_t wsb,
                                const ssm_mixer_stages* stages, hipStream_t stream) {
  g_err.clear();
  if (!stages) return fail(SSM_ERR_NULL, "mixer stages: stages is NULL");
  return mixer_run(c, w, u, out, batch, seqlen, add_residual, ws, wsb, stream, nullptr, nullptr, stages);
}

ssm_status ssm_mixer_step(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                          int64_t batch, float* state, float* conv_state, int32_t add_residual, void* ws, size_t wsb,
                          hipStream_t stream) {
  g_err.clear();
  if (batch > 0 && !state) return fail(SSM_ERR_NULL, "mixer step: state is NULL");
  if (batch > 0 && c && c->gated && c->d_conv > 1 && !conv_state)
    return fail(SSM_ERR_NULL, "mixer step: conv_state is NULL (gated block)");
  return mixer_run(c, w, u, out, batch, 1, add_residual, ws, wsb, stream, state, conv_state, nullptr);
}

size_t ssm_mixer_stack_workspace_bytes(const ssm_mixer_config* c, int64_t batch) {
  std::string keep = g_err;
  MixPlan p;
  const ssm_status st = mix_plan(c, batch, 1, &p);
  g_err = keep;
  if (st != SSM_OK) return 0;
  // the layer's workspace, then two [batch, d_model] activation buffers
  return align_up(ssm_mixer_workspace_bytes(c, batch, 1)) + 2 * align_up((size_t)batch * c->d_model * act_size(c->act_dtype));
}

ssm_status ssm_mixer_stack_step(const ssm_mixer_config* c, const ssm_mixer_weights* const* w, int32_t nlayers,
                                const void* u, void* out, int64_t batch, float* const* states,
                                float* const* conv_states, int32_t add_residual, void* ws, size_t wsb,
                                hipStream_t stream) {
  g_err.clear();
  MixPlan p;
  ssm_status st = mix_plan(c, batch, 1, &p);
  if (st != SSM_OK) return st;
  if (nlayers < 1) return fail(SSM_ERR_SHAPE, "mixer stack step: nlayers %d < 1", (int)nlayers);
  if (!w || !states) return fail(SSM_ERR_NULL, "mixer stack step: w and states are required");
  if (batch > 0 && (!u || !out)) return fail(SSM_ERR_NULL, "mixer stack step: u / out is NULL");
  if (out == u && !add_residual) return fail(SSM_ERR_SHAPE, "mixer stack step: out may alias u only with add_residual");
  const size_t need = ssm_mixer_stack_workspace_bytes(c, batch);
  if (!ws || wsb < need) return fail(SSM_ERR_WORKSPACE, "mixer stack step: workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(SSM_ERR_ALIGN, "mixer stack step: workspace must be 256-byte aligned");
  if (batch == 0) return SSM_OK;
  const size_t lwb = align_up(ssm_mixer_workspace_bytes(c, batch, 1));
  const size_t ab = align_up((size_t)batch * c->d_model * act_size(c->act_dtype));
  void* buf[2] = {(char*)ws + lwb, (char*)ws + lwb + ab};
  bool fused = true;
  for (int l = 0; l < nlayers && fused; ++l) fused = dec_layer_ok(c, w[l], states[l], batch, p.PW);
  if (fused) {  // the layers in launches of up to kDecMaxLayers, activations kept in LDS inside one
    for (int l0 = 0, g = 0; l0 < nlayers; l0 += kDecMaxLayers, ++g) {
      const int nl = nlayers - l0 < kDecMaxLayers ? nlayers - l0 : kDecMaxLayers;
      const void* in = l0 == 0 ? u : buf[(g - 1) % 2];
      void* o = l0 + nl == nlayers ? out : buf[g % 2];
      DecodeArgs da = dec_args(c, batch, p.PW, in, o, add_residual);
      da.nl = nl;
      for (int j = 0; j < nl; ++j) dec_layer(da.layer[j], w[l0 + j], states[l0 + j]);
      st = dev(launch_decode_m1(da, stream), "mixer stack step");
      if (st != SSM_OK) return st;
    }
    return SSM_OK;
  }
  // any other layer: ssm_mixer_step per layer, the activations between layers in the workspace
  for (int l = 0; l < nlayers; ++l) {
    const void* in = l == 0 ? u : buf[(l - 1) % 2];
    void* o = l + 1 == nlayers ? out : buf[l % 2];
    st = ssm_mixer_step(c, w[l], in, o, batch, states[l], conv_states ? conv_states[l] : nullptr, add_residual, ws,
                        lwb, stream);
    if (st != SSM_OK) return st;
  }
  return SSM_OK;
}

ssm_status ssm_conv1d_silu_fwd(const void* x, int32_t dtype, int64_t batch, int64_t seqlen, int64_t channels,
                               int64_t ldx, const float* w, int32_t width, const float* bias, const float* state_in,
                               float* state_out, void* out, int64_t ldo, hipStream_t stream) {
  g_err.clear();
  if (!act_dtype_ok(dtype)) return fail(SSM_ERR_DTYPE, "conv: dtype %d", dtype);
  if (batch < 0 || seqlen < 0 || channels < 1) return fail(SSM_ERR_SHAPE, "conv: batch, seqlen >= 0 and channels >= 1");
  if (width < 1 || width > kConvMaxK) return fail(SSM_ERR_SHAPE, "conv: width %d not in [1, %d]", (int)width, kConvMaxK);
  if (ldx < channels || ldo < channels) return fail(SSM_ERR_SHAPE, "conv: ldx / ldo < channels");
  if (batch * seqlen > 0 && (!x || !w || !out)) return fail(SSM_ERR_NULL, "conv: x, w and out are required");
  if (batch * seqlen > 0 && out == x) return fail(SSM_ERR_SHAPE, "conv: out may not alias x");
  ConvArgs a{};
  a.batch = batch; a.L = seqlen; a.C = channels; a.K = width; a.act_bf16 = dtype == SSM_BF16;
  a.x = x; a.ldx = ldx; a.w = w; a.bias = bias;
  a.state_in = width > 1 ? state_in : nullptr;
  a.state_out = width > 1 ? state_out : nullptr;
  a.out = out; a.ldo = ldo;
  return dev(launch_conv_silu(a, stream), "conv");
}

size_t ssm_selective_scan_bwd_workspace_bytes(const ssm_scan_bwd_args* a) {
  std::string keep = g_err;
  ScanBwdArgs s;
  const ssm_status st = scan_bwd_check(a, &s);
  g_err = keep;
  return st == SSM_OK ? scan_bwd_workspace(s) : 0;
}

ssm_status ssm_selective_scan_bwd(const ssm_scan_bwd_args* a, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  ScanBwdArgs s;
  ssm_status st = scan_bwd_check(a, &s);
  if (st != SSM_OK) return st;
  if (s.batch * s.L == 0) return SSM_OK;
  const size_t need = scan_bwd_workspace(s);
  if (!ws || wsb < need) return fail(SSM_ERR_WORKSPACE, "scan bwd: workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(SSM_ERR_ALIGN, "scan bwd: workspace must be 256-byte aligned");
  return dev(launch_scan_bwd(s, ws, stream), "scan bwd");
}

size_t ssm_bitlinear_bwd_workspace_bytes(const ssm_bitlinear_bwd_args* a) {
  std::string keep = g_err;
  SteArgs s;
  const ssm_status st = ste_check(a, &s);
  g_err = keep;
  return st == SSM_OK ? ste_workspace(s) : 0;
}

ssm_status ssm_bitlinear_bwd(const ssm_bitlinear_bwd_args* a, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  SteArgs s;
  ssm_status st = ste_check(a, &s);
  if (st != SSM_OK) return st;
  if (s.M == 0) return SSM_OK;
  const size_t need = ste_workspace(s);
  if (!ws || wsb < need) return fail(SSM_ERR_WORKSPACE, "bitlinear bwd: workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(SSM_ERR_ALIGN, "bitlinear bwd: workspace must be 256-byte aligned");
  return dev(launch_ste_bwd(s, ws, stream), "bitlinear bwd");
}

ssm_status ssm_qat_sgd_step(float* w_latent, float* w_scale, const float* dw, const float* d_scale, int64_t n_out,
                            int64_t k, int64_t group_size, float lr, float lr_scale, uint8_t* w_packed,
                            int64_t* zero_count, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  if (n_out < 1 || k < 1 || group_size < 0 || (group_size > 0 && (group_size % 64 != 0 || k % group_size != 0)))
    return fail(SSM_ERR_SHAPE, "qat step: n_out, k >= 1; group_size 0 or a multiple of 64 dividing k");
  if (!w_latent || !w_scale || !dw || !w_packed) return fail(SSM_ERR_NULL, "qat step: w_latent, w_scale, dw, w_packed");
  const int64_t ns = group_size ? n_out * (k / group_size) : 1;
  ssm_status st = dev(launch_sgd(w_latent, dw, n_out * k, lr, stream), "qat step weights");
  if (st != SSM_OK) return st;
  if (d_scale) {
    st = dev(launch_sgd(w_scale, d_scale, ns, lr_scale, stream), "qat step scales");
    if (st != SSM_OK) return st;
  }
  // the codes under the updated (learned) scales, with their zero count
  return ssm_ternary_quantize_weights(w_latent, n_out, k, group_size, w_scale, w_packed, w_scale, zero_count, ws, wsb,
                                      stream);
}

ssm_status ssm_dt_input_quantize(const void* dt_in, int32_t dtype, int64_t m, int64_t dt_rank, int64_t ld,
                                 const float* g_dt, float eps, int8_t* codes, double* deq, hipStream_t stream) {
  g_err.clear();
  if (!act_dtype_ok(dtype)) return fail(SSM_ERR_DTYPE, "dt quantize: dtype %d", dtype);
  if (m < 0) return fail(SSM_ERR_SHAPE, "dt quantize: m < 0");
  if (dt_rank < 1 || dt_rank > 64) return fail(SSM_ERR_UNSUPPORTED, "dt quantize: dt_rank must be in [1, 64]");
  if (ld < dt_rank) return fail(SSM_ERR_SHAPE, "dt quantize: ld < dt_rank");
  if (m > 0 && (!dt_in || !codes || !deq)) return fail(SSM_ERR_NULL, "dt quantize: dt_in, codes and deq are required");
  return dev(launch_dt_codes(dt_in, dtype == SSM_BF16, m, ld, (int)dt_rank, g_dt, eps, codes, deq, stream),
             "dt quantize");
}

ssm_status ssm_dense_fwd(const void* x, int32_t dtype, int64_t m, int64_t k, int64_t ldx, const void* w, int64_t n,
                         const void* residual, int64_t ld_res, void* y, int64_t ldy, hipStream_t stream) {
  g_err.clear();
  if (!act_dtype_ok(dtype)) return fail(SSM_ERR_DTYPE, "dense: dtype %d", dtype);
  const int64_t kMaxDim = 0x7fffffff;
  if (m < 0 || k < 1 || n < 1 || m > kMaxDim || k > kMaxDim || n > kMaxDim)
    return fail(SSM_ERR_SHAPE, "dense: m >= 0, k >= 1, n >= 1 (each below 2^31)");
  if (ldx < k || ldy < n || (residual && ld_res < n) || ldx > kMaxDim || ldy > kMaxDim)
    return fail(SSM_ERR_SHAPE, "dense: a row stride is smaller than its row");
  if (m > 0 && (!x || !w || !y)) return fail(SSM_ERR_NULL, "dense: x, w and y are required");
  if (m > 0 && x == y) return fail(SSM_ERR_SHAPE, "dense: y may not alias x");
  DenseArgs d{};
  d.M = m; d.N = n; d.K = k; d.bf16 = dtype == SSM_BF16;
  d.x = x; d.ldx = ldx; d.W = w; d.residual = residual; d.ld_res = ld_res; d.y = y; d.ldy = ldy;
  return dev(launch_dense(d, stream), "dense");
}

}  // extern "C"

namespace {
// Device-to-device copy of `rows` rows of `width` bytes (a stage output, for the checks).
ssm_status copy_rows(void* dst, const void* src, size_t src_pitch, size_t width, int64_t rows, hipStream_t stream) {
  if (!dst || rows == 0) return SSM_OK;
  return dev(hipMemcpy2DAsync(dst, width, src, src_pitch, width, (size_t)rows, hipMemcpyDeviceToDevice, stream),
             "mixer stage copy");
}

ssm_status mixer_run(const ssm_mixer_config* c, const ssm_mixer_weights* w, const void* u, void* out,
                     int64_t batch, int64_t seqlen, int32_t add_residual, void* ws, size_t wsb, hipStream_t stream,
                     float* state, float* conv_state, const ssm_mixer_stages* dbg) {
  MixPlan p;
  ssm_status st = mix_plan(c, batch, seqlen, &p);
  if (st != SSM_OK) return st;
  if (dbg) {
    const bool dt_stage = dbg->dt_codes || dbg->dt_deq || dbg->dt_acc;
    if (c->kind != SSM_MIXER_MAMBA1 && (dbg->x || dt_stage))
      return fail(SSM_ERR_UNSUPPORTED, "mixer stages: x and the dt stages exist for the Mamba-1 kind only");
    if (c->fp_proj == 2 && dt_stage)
      return fail(SSM_ERR_UNSUPPORTED, "mixer stages: the dt stages need the ternary dt projection (fp_proj < 2)");
  }
  // full-precision projections: in and out (fp_proj >= 1), x and dt too (fp_proj == 2)
  const bool f_io = c->fp_proj >= 1, f_xdt = c->fp_proj == 2;
  if (!w || !w->A) return fail(SSM_ERR_NULL, "mixer: weights and A are required");
  if (f_io ? (!w->fw_in || !w->fw_out) : (!w->w_in || !w->w_out || !w->s_in || !w->s_out))
    return fail(SSM_ERR_NULL, f_io ? "mixer: fw_in and fw_out are required (fp_proj >= 1)"
                                   : "mixer: w_in, w_out, s_in and s_out are required");
  if (c->kind == SSM_MIXER_MAMBA1 &&
      (f_xdt ? (!w->fw_x || !w->fw_dt) : (!w->w_x || !w->w_dt || !w->s_x || !w->s_dt)))
    return fail(SSM_ERR_NULL, f_xdt ? "mixer: fw_x and fw_dt are required (fp_proj == 2)"
                                    : "mixer: w_x, w_dt, s_x and s_dt are required for the Mamba-1 kind");
  if (c->gated && !w->conv_w) return fail(SSM_ERR_NULL, "mixer: conv_w is required for the gated block");
  if (p.M > 0 && (!u || !out)) return fail(SSM_ERR_NULL, "mixer: u / out is NULL");
  if (out == u && !add_residual) return fail(SSM_ERR_SHAPE, "mixer: out may alias u only with add_residual");
  const size_t need = ssm_mixer_workspace_bytes(c, batch, seqlen);
  if (!ws || wsb < need) return fail(SSM_ERR_WORKSPACE, "mixer: workspace needs %zu bytes", need);
  if (!aligned(ws, 256)) return fail(SSM_ERR_ALIGN, "mixer: workspace must be 256-byte aligned");
  if (p.M == 0) return SSM_OK;
  char* base = (char*)ws;
  float* am = (float*)(base + p.off_am);
  const size_t as = act_size(c->act_dtype);

  auto bitlinear = [&](const void* x, int64_t k, int64_t ldx, const uint8_t* wp, const float* sc, const float* g,
                       int64_t n, void* y, int64_t ldy, const void* res) -> ssm_status {
    ssm_bitlinear_args a{};
    a.x = x; a.x_dtype = c->act_dtype; a.act_bits = c->act_bits;
    a.m = p.M; a.k = k; a.ldx = ldx;
    a.norm_weight = g; a.norm_eps = c->norm_eps;
    a.w_packed = wp; a.w_scale = sc; a.n_out = n; a.group_size = c->group_size;
    a.residual = res; a.ld_res = c->d_model;
    a.y = y; a.y_dtype = c->act_dtype; a.ldy = ldy;
    BLPlan bp;
    ssm_status s2 = bl_plan(&a, &bp);
    if (s2 != SSM_OK) return s2;
    if (c->act_bits == 8 && !bp.rows) {  // tiled path: codes in the shared buffer, absmax in its own region
      a.dbg_absmax = am;
    }
    return bl_run(&a, bp, base, stream);
  };
  auto dense = [&](const void* x, int64_t k, int64_t ldx, const void* W, int64_t n, void* y, int64_t ldy,
                   const void* r) -> ssm_status {
    DenseArgs d{};
    d.M = p.M; d.N = n; d.K = k; d.bf16 = c->act_dtype == SSM_BF16;
    d.x = x; d.ldx = ldx; d.W = W; d.residual = r; d.ld_res = c->d_model; d.y = y; d.ldy = ldy;
    return dev(launch_dense(d, stream), "mixer dense projection");
  };
  // gated block: causal convolution + SiLU of the SSM input channels (Cc of them, row stride ld)
  auto conv = [&](const void* x, int64_t ld, void* xc) -> ssm_status {
    ConvArgs ca{};
    ca.batch = batch; ca.L = seqlen; ca.C = p.Cc; ca.K = (int)c->d_conv; ca.act_bf16 = c->act_dtype == SSM_BF16;
    ca.x = x; ca.ldx = ld; ca.w = w->conv_w; ca.bias = w->conv_b;
    ca.state_in = c->d_conv > 1 ? conv_state : nullptr;
    ca.state_out = c->d_conv > 1 ? conv_state : nullptr;
    ca.out = xc; ca.ldo = p.Cc;
    return dev(launch_conv_silu(ca, stream), "mixer conv");
  };

  const void* res = add_residual ? u : nullptr;
  if (c->kind == SSM_MIXER_MAMBA1) {
    void* xz = base + p.off_x;                         // in_proj output [x | zg]
    void* x = c->gated ? base + p.off_xc : xz;         // the SSM input
    void* pp = base + p.off_p;
    void* y = base + p.off_y;
    // one decoding step on a kernel of its own (a block per sequence runs the whole layer)
    if (seqlen == 1 && !dbg && dec_layer_ok(c, w, state, batch, p.PW)) {
      DecodeArgs da = dec_args(c, batch, p.PW, u, out, add_residual);
      da.nl = 1;
      dec_layer(da.layer[0], w, state);
      return dev(launch_decode_m1(da, stream), "mixer decode step");
    }
    const bool front = !c->gated && !c->fp_proj &&
                       front_supported((int)c->d_model, (int)c->d_inner, (int)p.PW, (int)c->dt_rank);
    ssm_scan_args sa{};
    sa.batch = batch; sa.seqlen = seqlen; sa.nheads = c->d_inner; sa.headdim = 1; sa.d_state = c->d_state;
    sa.a_per_state = 1; sa.act_dtype = c->act_dtype;
    sa.x = x; sa.ld_x = c->d_inner;
    sa.delta_bias = w->dt_bias; sa.delta_softplus = 1;
    sa.A = w->A;
    sa.Bm = (const char*)pp + c->dt_rank * as; sa.ld_B = p.PW;
    sa.Cm = (const char*)pp + (c->dt_rank + c->d_state) * as; sa.ld_C = p.PW;
    sa.D = w->D;
    sa.h0 = state; sa.h_last = state;
    sa.y = y; sa.ld_y = c->d_inner;
    if (f_xdt) {  // full-precision dt projection, stored, then read by the scan
      sa.delta = base + p.off_dl; sa.ld_delta = c->d_inner;
    } else {      // ternary dt projection inside the scan
      sa.dt_in = pp; sa.ld_dt_in = p.PW; sa.dt_rank = c->dt_rank;
      sa.w_dt = w->w_dt; sa.s_dt = w->s_dt; sa.g_dt = w->g_dt; sa.dt_eps = c->norm_eps;
    }
    if (c->gated) { sa.gate = (const char*)xz + c->d_inner * as; sa.ld_gate = p.XW; }
    st = scan_check(&sa);
    if (st != SSM_OK) return st;
    ScanArgs sc = to_scan(&sa);
    if (dbg) sc.dbg_dt_acc = dbg->dt_acc;
    if (p.off_scan + scan_m1_workspace(sc) > wsb)  // the scan's codes region lies inside the workspace
      return fail(SSM_ERR_WORKSPACE, "mixer: scan workspace exceeds %zu bytes", wsb);
    if (front) {  // in_proj, x_proj and the dt input's codes in one kernel, codes into the scan's workspace
      FrontArgs fa{};
      fa.M = p.M; fa.u = u; fa.act_bf16 = c->act_dtype == SSM_BF16;
      fa.Dm = (int)c->d_model; fa.Di = (int)c->d_inner; fa.PW = (int)p.PW; fa.R = (int)c->dt_rank;
      fa.w_in = (const uint32_t*)w->w_in; fa.s_in = w->s_in; fa.g_in = w->g_in;
      fa.w_x = (const uint32_t*)w->w_x; fa.s_x = w->s_x; fa.g_x = w->g_x;
      fa.eps = c->norm_eps; fa.x = x; fa.p = pp; fa.g_dt = w->g_dt;
      size_t off_deq = 0;
      scan_m1_code_layout(sc, &fa.cw, &off_deq);
      fa.codes = (int8_t*)(base + p.off_scan);
      fa.deq = (double*)(base + p.off_scan + off_deq);
      st = dev(launch_m1_front(fa, stream), "mixer front");
      if (st != SSM_OK) return st;
      sc.dt_codes_ready = 1;
    } else {
      st = f_io ? dense(u, c->d_model, c->d_model, w->fw_in, p.XW, xz, p.XW, nullptr)
                : bitlinear(u, c->d_model, c->d_model, w->w_in, w->s_in, w->g_in, p.XW, xz, p.XW, nullptr);
      if (st != SSM_OK) return st;
      if (c->gated) {
        st = conv(xz, p.XW, x);
        if (st != SSM_OK) return st;
      }
      st = f_xdt ? dense(x, c->d_inner, c->d_inner, w->fw_x, p.PW, pp, p.PW, nullptr)
                 : bitlinear(x, c->d_inner, c->d_inner, w->w_x, w->s_x, w->g_x, p.PW, pp, p.PW, nullptr);
      if (st != SSM_OK) return st;
      if (f_xdt) {
        st = dense(pp, c->dt_rank, p.PW, w->fw_dt, c->d_inner, base + p.off_dl, c->d_inner, nullptr);
        if (st != SSM_OK) return st;
      }
    }
    st = dev(launch_scan_m1(sc, base + p.off_scan, stream), "mixer scan");
    if (st != SSM_OK) return st;
    if (dbg) {  // the stages as the kernels left them in the workspace (before out_proj runs)
      int cw = 0;
      size_t off_deq = 0;
      scan_m1_code_layout(sc, &cw, &off_deq);
      ssm_status e = copy_rows(dbg->x, x, c->d_inner * as, c->d_inner * as, p.M, stream);
      if (e == SSM_OK) e = copy_rows(dbg->p, pp, p.PW * as, p.PW * as, p.M, stream);
      if (e == SSM_OK) e = copy_rows(dbg->dt_codes, base + p.off_scan, cw, c->dt_rank, p.M, stream);
      if (e == SSM_OK) e = copy_rows(dbg->dt_deq, base + p.off_scan + off_deq, 8, 8, p.M, stream);
      if (e == SSM_OK) e = copy_rows(dbg->y, y, c->d_inner * as, c->d_inner * as, p.M, stream);
      if (e != SSM_OK) return e;
    }
    return f_io ? dense(y, c->d_inner, c->d_inner, w->fw_out, c->d_model, out, c->d_model, res)
                : bitlinear(y, c->d_inner, c->d_inner, w->w_out, w->s_out, w->g_out, c->d_model, out, c->d_model, res);
  }
  // SSD kind: v = [x | B | C | dt (| zg)]; the gated block reads x, B and C from their convolution
  void* v = base + p.off_p;
  void* y = base + p.off_y;
  st = f_io ? dense(u, c->d_model, c->d_model, w->fw_in, p.VW, v, p.VW, nullptr)
            : bitlinear(u, c->d_model, c->d_model, w->w_in, w->s_in, w->g_in, p.VW, v, p.VW, nullptr);
  if (st != SSM_OK) return st;
  const void* xbc = v;
  int64_t ld_xbc = p.VW;
  if (c->gated) {
    st = conv(v, p.VW, base + p.off_xc);
    if (st != SSM_OK) return st;
    xbc = base + p.off_xc;
    ld_xbc = p.Cc;
  }
  ScanArgs s{};
  s.batch = batch; s.L = seqlen; s.H = c->nheads; s.P = c->headdim; s.N = c->d_state;
  s.act_bf16 = c->act_dtype == SSM_BF16;
  s.x = xbc; s.ld_x = ld_xbc;
  s.Bm = (const char*)xbc + c->d_inner * as; s.ld_B = ld_xbc;
  s.Cm = (const char*)xbc + (c->d_inner + c->d_state) * as; s.ld_C = ld_xbc;
  s.delta = (const char*)v + (c->d_inner + 2 * c->d_state) * as; s.ld_delta = p.VW;
  s.delta_bias = w->dt_bias; s.softplus = 1;
  s.A = w->A; s.D = w->D;
  s.h0 = state; s.h_last = state;
  s.y = y; s.ld_y = c->d_inner;
  if (c->gated) { s.gate = (const char*)v + p.VW0 * as; s.ld_gate = p.VW; }
  st = dev(launch_scan_ssd(s, base + p.off_scan, wsb - p.off_scan, stream), "mixer scan");
  if (st != SSM_OK) return st;
  if (dbg) {
    ssm_status e = copy_rows(dbg->p, v, p.VW * as, p.VW * as, p.M, stream);
    if (e == SSM_OK) e = copy_rows(dbg->y, y, c->d_inner * as, c->d_inner * as, p.M, stream);
    if (e != SSM_OK) return e;
  }
  return f_io ? dense(y, c->d_inner, c->d_inner, w->fw_out, c->d_model, out, c->d_model, res)
              : bitlinear(y, c->d_inner, c->d_inner, w->w_out, w->s_out, w->g_out, c->d_model, out, c->d_model, res);
}

}  // namespace

// ------------------------------------------------------------------ mixer backward

namespace {
// Workspace of the mixer backward: the forward's intermediates (x, p, delta, y), the chain's
// gradients (dy of the scan output, dx through the scan, d delta, dB, dC, the x_proj output's
// gradient, dx through x_proj, a dA scratch) and one sub-workspace that the steps take in turn.
struct MixBwdPlan {
  int64_t M = 0, PW = 0;
  size_t off_x = 0, off_p = 0, off_dl = 0, off_y = 0, off_dy = 0, off_dxs = 0, off_ddl = 0, off_dB = 0,
         off_dC = 0, off_dA = 0, off_dp = 0, off_sub = 0, total = 0;
};

ssm_status mixer_bwd_plan(const ssm_mixer_config* c, int64_t batch, int64_t seqlen, MixBwdPlan* p) {
  MixPlan mp;
  ssm_status st = mix_plan(c, batch, seqlen, &mp);
  if (st != SSM_OK) return st;
  if (c->kind != SSM_MIXER_MAMBA1 || c->gated || c->fp_proj || c->act_dtype != SSM_F32)
    return fail(SSM_ERR_UNSUPPORTED, "mixer bwd: Mamba-1 kind, not gated, ternary projections, fp32 activations");
  {  // the scan backward's own limits, checked here so that the workspace size is only given for runnable shapes
    ssm_scan_bwd_args q{};
    q.batch = batch; q.seqlen = seqlen; q.nheads = c->d_inner; q.d_state = c->d_state; q.act_dtype = SSM_F32;
    q.ld_x = q.ld_delta = q.ld_dy = c->d_inner; q.ld_B = q.ld_C = c->d_state;
    const uintptr_t nz = 256;  // stand-ins for the buffers the call itself provides (never dereferenced)
    q.x = q.delta = q.Bm = q.Cm = (const void*)nz;
    q.A = q.dy = (const float*)nz;
    q.dx = q.ddelta = q.dA = q.dB = q.dC = (float*)nz;
    ScanBwdArgs tmp;
    st = scan_bwd_check(&q, &tmp);
    if (st != SSM_OK) return st;
  }
  const int64_t M = batch * seqlen, Dm = c->d_model, Di = c->d_inner, N = c->d_state, R = c->dt_rank;
  p->M = M;
  p->PW = mp.PW;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  p->off_x = take((size_t)M * Di * 4);
  p->off_p = take((size_t)M * p->PW * 4);
  p->off_dl = take((size_t)M * Di * 4);
  p->off_y = take((size_t)M * Di * 4);
  p->off_dy = take((size_t)M * Di * 4);
  p->off_dxs = take((size_t)M * Di * 4);
  p->off_ddl = take((size_t)M * Di * 4);
  p->off_dB = take((size_t)M * N * 4);
  p->off_dC = take((size_t)M * N * 4);
  p->off_dA = take((size_t)Di * N * 4);
  p->off_dp = take((size_t)M * p->PW * 4);
  p->off_sub = off;
  // the largest of the steps' own workspaces (sizes depend on shapes only)
  size_t sub = 0;
  auto bl_ws = [&](int64_t k, int64_t n) {
    ssm_bitlinear_args a{};
    a.x_dtype = SSM_F32; a.act_bits = 8; a.m = M; a.k = k; a.ldx = k; a.n_out = n; a.y_dtype = SSM_F32; a.ldy = n;
    a.w_packed = (const uint8_t*)(uintptr_t)256; a.w_scale = (const float*)(uintptr_t)256;
    BLPlan bp;
    if (bl_plan(&a, &bp) == SSM_OK && bp.total > sub) sub = bp.total;
  };
  bl_ws(Dm, Di);
  bl_ws(Di, p->PW);
  bl_ws(R, Di);
  ScanArgs sa{};
  sa.batch = batch; sa.L = seqlen; sa.H = Di; sa.P = 1; sa.N = N;
  sub = std::max(sub, scan_m1_workspace(sa));
  ScanBwdArgs sb{};
  sb.batch = batch; sb.L = seqlen; sb.H = Di; sb.N = N;
  sub = std::max(sub, scan_bwd_workspace(sb));
  auto ste_ws = [&](int64_t k, int64_t n) {
    SteArgs s2{};
    s2.M = M; s2.K = k; s2.N = n;
    sub = std::max(sub, ste_workspace(s2));
  };
  ste_ws(Di, Dm);
  ste_ws(R, Di);
  ste_ws(Di, p->PW);
  ste_ws(Dm, Di);
  p->total = off + align_up(sub);
  return SSM_OK;
}
}  // namespace

extern "C" {

size_t ssm_mixer_bwd_workspace_bytes(const ssm_mixer_config* c, int64_t batch, int64_t seqlen) {
  std::string keep = g_err;
  MixBwdPlan p;
  const ssm_status st = mixer_bwd_plan(c, batch, seqlen, &p);
  g_err = keep;
  return st == SSM_OK ? p.total : 0;
}

ssm_status ssm_mixer_bwd(const ssm_mixer_config* c, const ssm_mixer_weights* w, const ssm_mixer_grads* g,
                         const float* u, const float* dout, float* du, int64_t batch, int64_t seqlen,
                         int32_t add_residual, void* ws, size_t wsb, hipStream_t stream) {
  g_err.clear();
  MixBwdPlan p;
  ssm_status st = mixer_bwd_plan(c, batch, seqlen, &p);
  if (st != SSM_OK) return st;
  if (!w || !w->A || !w->w_in || !w->w_x || !w->w_dt || !w->w_out || !w->s_in || !w->s_x || !w->s_dt || !w->s_out)
    return fail(SSM_ERR_NULL, "mixer bwd: w_in, w_x, w_dt, w_out, their scales and A are required");
  const ssm_mixer_grads none{};
  const ssm_mixer_grads& gr = g ? *g : none;
  if ((gr.ds_in && (!gr.dw_in || !gr.lat_in)) || (gr.ds_x && (!gr.dw_x || !gr.lat_x)) ||
      (gr.ds_dt && (!gr.dw_dt || !gr.lat_dt)) || (gr.ds_out && (!gr.dw_out || !gr.lat_out)))
    return fail(SSM_ERR_NULL, "mixer bwd: a scale gradient needs its dw and the latent weights");
  if (p.M > 0 && (!u || !dout || !du)) return fail(SSM_ERR_NULL, "mixer bwd: u, dout and du are required");
  if (p.M > 0 && ((const void*)du == (const void*)u || du == dout))
    return fail(SSM_ERR_SHAPE, "mixer bwd: du may not alias u or dout");
  if (!ws || wsb < p.total) return fail(SSM_ERR_WORKSPACE, "mixer bwd: workspace needs %zu bytes", p.total);
  if (!aligned(ws, 256)) return fail(SSM_ERR_ALIGN, "mixer bwd: workspace must be 256-byte aligned");
  if (p.M == 0) return SSM_OK;
  char* base = (char*)ws;
  void* sub = base + p.off_sub;
  const int64_t M = p.M, Dm = c->d_model, Di = c->d_inner, N = c->d_state, R = c->dt_rank, PW = p.PW;
  float* x = (float*)(base + p.off_x);
  float* pp = (float*)(base + p.off_p);
  float* dl = (float*)(base + p.off_dl);
  float* y = (float*)(base + p.off_y);
  float* dy = (float*)(base + p.off_dy);
  float* dxs = (float*)(base + p.off_dxs);
  float* ddl = (float*)(base + p.off_ddl);
  float* dB = (float*)(base + p.off_dB);
  float* dC = (float*)(base + p.off_dC);
  float* dp = (float*)(base + p.off_dp);

  // ---- forward again, keeping x, p, delta and y
  auto bitlinear = [&](const void* xin, int64_t k, int64_t ldx, const uint8_t* wp, const float* sc, const float* gn,
                       int64_t n, float* out, int64_t ldy) -> ssm_status {
    ssm_bitlinear_args a{};
    a.x = xin; a.x_dtype = SSM_F32; a.act_bits = 8;
    a.m = M; a.k = k; a.ldx = ldx;
    a.norm_weight = gn; a.norm_eps = c->norm_eps;
    a.w_packed = wp; a.w_scale = sc; a.n_out = n; a.group_size = 0;
    a.y = out; a.y_dtype = SSM_F32; a.ldy = ldy;
    BLPlan bp;
    ssm_status s2 = bl_plan(&a, &bp);
    if (s2 != SSM_OK) return s2;
    return bl_run(&a, bp, sub, stream);
  };
  st = bitlinear(u, Dm, Dm, w->w_in, w->s_in, w->g_in, Di, x, Di);
  if (st != SSM_OK) return st;
  st = bitlinear(x, Di, Di, w->w_x, w->s_x, w->g_x, PW, pp, PW);
  if (st != SSM_OK) return st;
  st = bitlinear(pp, R, PW, w->w_dt, w->s_dt, w->g_dt, Di, dl, Di);
  if (st != SSM_OK) return st;
  ssm_scan_args sa{};
  sa.batch = batch; sa.seqlen = seqlen; sa.nheads = Di; sa.headdim = 1; sa.d_state = N;
  sa.a_per_state = 1; sa.act_dtype = SSM_F32;
  sa.x = x; sa.ld_x = Di;
  sa.delta = dl; sa.ld_delta = Di; sa.delta_bias = w->dt_bias; sa.delta_softplus = 1;
  sa.A = w->A;
  sa.Bm = pp + R; sa.ld_B = PW;
  sa.Cm = pp + R + N; sa.ld_C = PW;
  sa.D = w->D;
  sa.y = y; sa.ld_y = Di;
  st = scan_check(&sa);
  if (st != SSM_OK) return st;
  st = dev(launch_scan_m1(to_scan(&sa), sub, stream), "mixer bwd: scan");
  if (st != SSM_OK) return st;

  // ---- the chain, backwards
  auto bl_bwd = [&](const float* xin, int64_t k, int64_t ldx, const uint8_t* wp, const float* sc, const float* gn,
                    const float* lat, int64_t n, const float* gy, int64_t ld_gy, float* gx, int64_t ld_gx,
                    float* dw, float* ds, const float* add, int64_t ld_add) -> ssm_status {
    ssm_bitlinear_bwd_args a{};
    a.x = xin; a.x_dtype = SSM_F32; a.m = M; a.k = k; a.ldx = ldx;
    a.norm_weight = gn; a.norm_eps = c->norm_eps;
    a.w_packed = wp; a.w_scale = sc; a.n_out = n; a.group_size = 0;
    a.w_latent = lat;
    a.dy = gy; a.ld_dy = ld_gy;
    a.dx = gx; a.ld_dx = ld_gx;
    a.dw = dw; a.d_scale = ds;
    SteArgs s2;
    const ssm_status s3 = ste_check(&a, &s2);
    if (s3 != SSM_OK) return s3;
    return dev(launch_ste_bwd_add(s2, add, ld_add, sub, stream), "mixer bwd: bitlinear bwd");
  };
  st = bl_bwd(y, Di, Di, w->w_out, w->s_out, w->g_out, gr.lat_out, Dm, dout, Dm, dy, Di, gr.dw_out, gr.ds_out,
              nullptr, 0);
  if (st != SSM_OK) return st;
  ssm_scan_bwd_args qa{};
  qa.batch = batch; qa.seqlen = seqlen; qa.nheads = Di; qa.d_state = N;
  qa.act_dtype = SSM_F32; qa.delta_softplus = 1;
  qa.x = x; qa.ld_x = Di;
  qa.delta = dl; qa.ld_delta = Di;
  qa.delta_bias = w->dt_bias; qa.A = w->A;
  qa.Bm = pp + R; qa.ld_B = PW;
  qa.Cm = pp + R + N; qa.ld_C = PW;
  qa.D = w->D; qa.h0 = nullptr;
  qa.dy = dy; qa.ld_dy = Di;
  qa.dx = dxs; qa.ddelta = ddl;
  qa.dA = gr.dA ? gr.dA : (float*)(base + p.off_dA);
  qa.dB = dB; qa.dC = dC;
  qa.dD = gr.dD; qa.dbias = gr.d_dt_bias; qa.dh0 = nullptr;
  ScanBwdArgs sb;
  st = scan_bwd_check(&qa, &sb);
  if (st != SSM_OK) return st;
  st = dev(launch_scan_bwd(sb, sub, stream), "mixer bwd: scan bwd");
  if (st != SSM_OK) return st;
  // d dr into the first R columns of the x_proj output's gradient, then dB and dC
  st = bl_bwd(pp, R, PW, w->w_dt, w->s_dt, w->g_dt, gr.lat_dt, Di, ddl, Di, dp, PW, gr.dw_dt, gr.ds_dt, nullptr, 0);
  if (st != SSM_OK) return st;
  st = dev(launch_copy_cols(dB, M, N, dp + R, PW, stream), "mixer bwd: dB");
  if (st != SSM_OK) return st;
  st = dev(launch_copy_cols(dC, M, N, dp + R + N, PW, stream), "mixer bwd: dC");
  if (st != SSM_OK) return st;
  // dx = dx_s + x_proj's dx, accumulated in place; du = in_proj's dx (+ dout)
  st = bl_bwd(x, Di, Di, w->w_x, w->s_x, w->g_x, gr.lat_x, PW, dp, PW, dxs, Di, gr.dw_x, gr.ds_x, dxs, Di);
  if (st != SSM_OK) return st;
  return bl_bwd(u, Dm, Dm, w->w_in, w->s_in, w->g_in, gr.lat_in, Di, dxs, Di, du, Dm, gr.dw_in, gr.ds_in,
                add_residual ? dout : nullptr, Dm);
}

}  // extern "C"
