// Host side of Floyd attention (include/fa_floyd.h): validation against the
// shape rules of page "CANN Floyd注意力梯度算子" (section 约束说明), the
// workspace layout and the launch sequence of the forward and the backward.
// Plain C++; the kernels are in fa_floyd_kernels.hip.

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>

#include "fa_floyd.h"
#include "fa_floyd_internal.h"

namespace {

using namespace ffloyd;

constexpr uint64_t kChunkCap = 4ull << 30;  // workspace budget for a group of heads
constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  int64_t NMK, NMD, NKD, KMD, NM, MK, MD, KD;
  int64_t heads;  // B * H
  int64_t hc;     // heads per chunk
  // byte offsets inside the workspace
  uint64_t o_s, o_p, o_pe, o_dse, o_dq, o_sfmg, o_lse2, total;
};

int plan(const fa_floyd_desc* d, Layout* L) {
  if (!d) return FA_ERR_NULLPTR;
  if (d->abi_version != FA_BWD_ABI_VERSION) return FA_ERR_PARAM_INVALID;
  if (d->dtype != FA_DTYPE_BF16 && d->dtype != FA_DTYPE_FP16) return FA_ERR_PARAM_INVALID;
  if (!std::isfinite(d->scale_value)) return FA_ERR_PARAM_INVALID;
  const int64_t lim = 1 << 20;
  if (d->B < 1 || d->B > 2048 || d->H < 1 || d->H > 256) return FA_ERR_SHAPE;
  if (d->N < 16 || d->N > lim || d->N % 16) return FA_ERR_SHAPE;
  if (d->M < 128 || d->M > lim || d->M % 128) return FA_ERR_SHAPE;
  if (d->K < 128 || d->K > lim || d->K % 128) return FA_ERR_SHAPE;
  if (d->D != 32 && d->D != 64 && d->D != 128) return FA_ERR_SHAPE;
  const int64_t N = d->N, M = d->M, K = d->K, D = d->D;
  L->MK = M * K;
  L->MD = M * D;
  L->KD = K * D;
  L->NM = N * M;
  L->NMD = N * M * D;
  L->NKD = N * K * D;
  L->KMD = K * M * D;
  // one head's fp32 score workspace must be addressable and its launches'
  // grids within 2^31 workgroups (x) and 65535 (heads, y)
  if ((double)N * M * K > (double)(1ll << 40)) return FA_ERR_UNSUPPORTED;
  L->NMK = N * M * K;
  const int64_t t128 = 128;
  const int64_t grid_x[] = {((M + t128 - 1) / t128) * ((K + t128 - 1) / t128) * N,
                            ((N + t128 - 1) / t128) * ((K + t128 - 1) / t128) * M,
                            ((K + t128 - 1) / t128) * N, ((K + t128 - 1) / t128) * M,
                            ((M + t128 - 1) / t128) * N, ((N + t128 - 1) / t128) * M};
  for (int64_t g : grid_x)
    if (g > 0x7fffffffll) return FA_ERR_UNSUPPORTED;
  L->heads = (int64_t)d->B * d->H;
  const uint64_t per_head = (uint64_t)L->NMK * 12 + (uint64_t)L->NMD * 4 + (uint64_t)L->NM * 8 + 7 * kAlign;
  uint64_t cap = kChunkCap;
  if (const char* e = std::getenv("FA_FLOYD_CHUNK_BYTES")) {
    const unsigned long long v = std::strtoull(e, nullptr, 10);
    if (v > 0) cap = v;
  }
  int64_t hc = (int64_t)(cap / per_head);
  if (hc < 1) hc = 1;
  if (hc > L->heads) hc = L->heads;
  if (hc > 65535) hc = 65535;
  L->hc = hc;
  uint64_t o = 0;
  L->o_s = o;    o = align_up(o + (uint64_t)hc * L->NMK * 4);
  L->o_p = o;    o = align_up(o + (uint64_t)hc * L->NMK * 4);
  L->o_pe = o;   o = align_up(o + (uint64_t)hc * L->NMK * 2);
  L->o_dse = o;  o = align_up(o + (uint64_t)hc * L->NMK * 2);
  L->o_dq = o;   o = align_up(o + (uint64_t)hc * L->NMD * 4);
  L->o_sfmg = o; o = align_up(o + (uint64_t)hc * L->NM * 4);
  L->o_lse2 = o; o = align_up(o + (uint64_t)hc * L->NM * 4);
  L->total = o;
  return FA_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
const T* at(const void* p, int64_t elems) {
  return static_cast<const T*>(p) + elems;
}
template <typename T>
T* at(void* p, int64_t elems) {
  return static_cast<T*>(p) + elems;
}

// 16-bit elements
const uint16_t* e16(const void* p, int64_t off) { return at<uint16_t>(p, off); }
uint16_t* e16(void* p, int64_t off) { return at<uint16_t>(p, off); }

GemmArgs gemm_base(const fa_floyd_desc* d, int64_t hc) {
  GemmArgs g{};
  g.heads = (int32_t)hc;
  g.f16 = d->dtype == FA_DTYPE_FP16;
  return g;
}

int bwd(const fa_floyd_desc* d, const void* query, const void* key1, const void* value1, const void* key2,
        const void* value2, const void* dy, const uint8_t* atten_mask, const float* softmax_max,
        const float* softmax_sum, const void* attention_in, void* dq, void* dk1, void* dv1, void* dk2, void* dv2,
        void* workspace, size_t workspace_bytes, void* stream, float* stage_ms);

}  // namespace

extern "C" {

int fa_floyd_workspace_size(const fa_floyd_desc* desc, size_t* workspace_bytes) {
  if (!workspace_bytes) return FA_ERR_NULLPTR;
  Layout L;
  const int rc = plan(desc, &L);
  if (rc != FA_OK) return rc;
  *workspace_bytes = (size_t)L.total;
  return FA_OK;
}

int fa_floyd_bwd_run(const fa_floyd_desc* d, const void* query, const void* key1, const void* value1,
                     const void* key2, const void* value2, const void* dy, const uint8_t* atten_mask,
                     const float* softmax_max, const float* softmax_sum, const void* attention_in, void* dq,
                     void* dk1, void* dv1, void* dk2, void* dv2, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return bwd(d, query, key1, value1, key2, value2, dy, atten_mask, softmax_max, softmax_sum, attention_in, dq, dk1,
             dv1, dk2, dv2, workspace, workspace_bytes, stream, nullptr);
}

int fa_floyd_bwd_run_timed(const fa_floyd_desc* d, const void* query, const void* key1, const void* value1,
                           const void* key2, const void* value2, const void* dy, const uint8_t* atten_mask,
                           const float* softmax_max, const float* softmax_sum, const void* attention_in, void* dq,
                           void* dk1, void* dv1, void* dk2, void* dv2, void* workspace, size_t workspace_bytes,
                           void* stream, float* stage_ms) {
  if (!stage_ms) return FA_ERR_NULLPTR;
  return bwd(d, query, key1, value1, key2, value2, dy, atten_mask, softmax_max, softmax_sum, attention_in, dq, dk1,
             dv1, dk2, dv2, workspace, workspace_bytes, stream, stage_ms);
}

}  // extern "C"

namespace {

int bwd(const fa_floyd_desc* d, const void* query, const void* key1, const void* value1, const void* key2,
        const void* value2, const void* dy, const uint8_t* atten_mask, const float* softmax_max,
        const float* softmax_sum, const void* attention_in, void* dq, void* dk1, void* dv1, void* dk2, void* dv2,
        void* workspace, size_t workspace_bytes, void* stream, float* stage_ms) {
  Layout L;
  int rc = plan(d, &L);
  if (rc != FA_OK) return rc;
  const void* in[] = {query, key1, value1, key2, value2, dy, softmax_max, softmax_sum, attention_in,
                      dq, dk1, dv1, dk2, dv2};
  for (const void* p : in) {
    if (!p) return FA_ERR_NULLPTR;
    if (!aligned(p)) return FA_ERR_PARAM_INVALID;
  }
  if (!workspace || workspace_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned(workspace)) return FA_ERR_PARAM_INVALID;
  char* ws = static_cast<char*>(workspace);
  float* ws_s = reinterpret_cast<float*>(ws + L.o_s);
  float* ws_p = reinterpret_cast<float*>(ws + L.o_p);
  void* ws_pe = ws + L.o_pe;
  void* ws_dse = ws + L.o_dse;
  float* ws_dq = reinterpret_cast<float*>(ws + L.o_dq);
  float* ws_sfmg = reinterpret_cast<float*>(ws + L.o_sfmg);
  float* ws_lse2 = reinterpret_cast<float*>(ws + L.o_lse2);
  const float scale = d->scale_value;
  const int f16 = d->dtype == FA_DTYPE_FP16;
  const int64_t chunks = (L.heads + L.hc - 1) / L.hc;
  StageTimer* timer = nullptr;
  int mark = 0;
  if (stage_ms) {
    timer = stage_timer_create((int)(chunks * FA_FLOYD_BWD_STAGES + 1));
    if (!timer) return FA_ERR_RUNTIME;
  }
  // a mark before the first stage and after each one (timed runs only)
  auto tick = [&]() { return timer ? stage_timer_mark(timer, mark++, stream) : 0; };
  auto fail = [&]() {
    stage_timer_destroy(timer);
    return FA_ERR_RUNTIME;
  };
  if (tick()) return fail();

  for (int64_t h0 = 0; h0 < L.heads; h0 += L.hc) {
    const int64_t hc = L.heads - h0 < L.hc ? L.heads - h0 : L.hc;
    const void* q = e16(query, h0 * L.NMD);
    const void* g = e16(dy, h0 * L.NMD);
    const void* y = e16(attention_in, h0 * L.NMD);
    const void* k1 = e16(key1, h0 * L.NKD);
    const void* v1 = e16(value1, h0 * L.NKD);
    const void* k2 = e16(key2, h0 * L.KMD);
    const void* v2 = e16(value2, h0 * L.KMD);

    RowStatsArgs r{};
    r.dy = g;
    r.y = y;
    r.smax = softmax_max + h0 * L.NM * 8;
    r.ssum = softmax_sum + h0 * L.NM * 8;
    r.sfmg = ws_sfmg;
    r.lse2 = ws_lse2;
    r.rows = hc * L.NM;
    r.D = d->D;
    r.f16 = f16;
    if (launch_rowstats(r, stream)) return fail();
    if (tick()) return fail();

    ScoreArgs s{};
    s.q = q;
    s.dy = g;
    s.ws_s = ws_s;
    s.ws_p = ws_p;
    s.ws_pe = ws_pe;
    s.ws_dse = ws_dse;
    s.sfmg = ws_sfmg;
    s.lse2 = ws_lse2;
    s.mask = atten_mask;
    s.head0 = (int32_t)h0;
    s.heads = (int32_t)hc;
    s.H = d->H;
    s.N = d->N;
    s.M = d->M;
    s.K = d->K;
    s.D = d->D;
    s.scale = scale;
    s.f16 = f16;
    s.x1 = k1;
    s.x2 = v1;
    s.by_m = 0;
    s.epi = 0;
    if (launch_scores(s, stream)) return fail();
    if (tick()) return fail();
    s.x1 = k2;
    s.x2 = v2;
    s.by_m = 1;
    s.epi = 1;
    if (launch_scores(s, stream)) return fail();
    if (tick()) return fail();

    // dV1 = P^T dY and dK1 = scale dS^T Q, batched over n: C(k, d), contraction over m
    GemmArgs a = gemm_base(d, hc);
    a.a_si = 1; a.a_st = d->K; a.a_sh = L.NMK; a.a_sz = L.MK; a.a_tc = 0;
    a.b_sj = 1; a.b_st = d->D; a.b_sh = L.NMD; a.b_sz = L.MD; a.b_tc = 0;
    a.c_si = d->D; a.c_sh = L.NKD; a.c_sz = L.KD;
    a.I = d->K; a.J = d->D; a.T = d->M; a.nb = d->N;
    a.a = ws_pe; a.b = g; a.c = e16(dv1, h0 * L.NKD); a.alpha = 1.f;
    if (launch_gemm(a, stream)) return fail();
    if (tick()) return fail();
    a.a = ws_dse; a.b = q; a.c = e16(dk1, h0 * L.NKD); a.alpha = scale;
    if (launch_gemm(a, stream)) return fail();
    if (tick()) return fail();

    // dV2 and dK2, batched over m: C(k, d) at [k][m][d], contraction over n
    GemmArgs b = gemm_base(d, hc);
    b.a_si = 1; b.a_st = L.MK; b.a_sh = L.NMK; b.a_sz = d->K; b.a_tc = 0;
    b.b_sj = 1; b.b_st = L.MD; b.b_sh = L.NMD; b.b_sz = d->D; b.b_tc = 0;
    b.c_si = L.MD; b.c_sh = L.KMD; b.c_sz = d->D;
    b.I = d->K; b.J = d->D; b.T = d->N; b.nb = d->M;
    b.a = ws_pe; b.b = g; b.c = e16(dv2, h0 * L.KMD); b.alpha = 1.f;
    if (launch_gemm(b, stream)) return fail();
    if (tick()) return fail();
    b.a = ws_dse; b.b = q; b.c = e16(dk2, h0 * L.KMD); b.alpha = scale;
    if (launch_gemm(b, stream)) return fail();
    if (tick()) return fail();

    // dQ: scale dS K1 (batched over n, fp32 partial), then + scale dS K2 (batched over m)
    GemmArgs c = gemm_base(d, hc);
    c.a_si = d->K; c.a_st = 1; c.a_sh = L.NMK; c.a_sz = L.MK; c.a_tc = 1;
    c.b_sj = 1; c.b_st = d->D; c.b_sh = L.NKD; c.b_sz = L.KD; c.b_tc = 0;
    c.c_si = d->D; c.c_sh = L.NMD; c.c_sz = L.MD;
    c.I = d->M; c.J = d->D; c.T = d->K; c.nb = d->N;
    c.a = ws_dse; c.b = k1; c.c = ws_dq; c.out_f32 = 1; c.alpha = scale;
    if (launch_gemm(c, stream)) return fail();
    if (tick()) return fail();
    GemmArgs e = gemm_base(d, hc);
    e.a_si = L.MK; e.a_st = 1; e.a_sh = L.NMK; e.a_sz = d->K; e.a_tc = 1;
    e.b_sj = 1; e.b_st = L.MD; e.b_sh = L.KMD; e.b_sz = d->D; e.b_tc = 0;
    e.c_si = L.MD; e.c_sh = L.NMD; e.c_sz = d->D;
    e.I = d->N; e.J = d->D; e.T = d->K; e.nb = d->M;
    e.a = ws_dse; e.b = k2; e.c = e16(dq, h0 * L.NMD); e.addend = ws_dq; e.alpha = scale;
    if (launch_gemm(e, stream)) return fail();
    if (tick()) return fail();
  }
  if (timer) {
    std::vector<float> ms((size_t)chunks * FA_FLOYD_BWD_STAGES);
    const int rc = stage_timer_read(timer, ms.data());
    stage_timer_destroy(timer);
    if (rc) return FA_ERR_RUNTIME;
    for (int i = 0; i < FA_FLOYD_BWD_STAGES; ++i) stage_ms[i] = 0.f;
    for (size_t i = 0; i < ms.size(); ++i) stage_ms[i % FA_FLOYD_BWD_STAGES] += ms[i];
  }
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_floyd_fwd_run(const fa_floyd_desc* d, const void* query, const void* key1, const void* value1,
                     const void* key2, const void* value2, const uint8_t* atten_mask, void* attention_out,
                     float* softmax_max, float* softmax_sum, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Layout L;
  int rc = plan(d, &L);
  if (rc != FA_OK) return rc;
  const void* in[] = {query, key1, value1, key2, value2, attention_out, softmax_max, softmax_sum};
  for (const void* p : in) {
    if (!p) return FA_ERR_NULLPTR;
    if (!aligned(p)) return FA_ERR_PARAM_INVALID;
  }
  if (!workspace || workspace_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned(workspace)) return FA_ERR_PARAM_INVALID;
  char* ws = static_cast<char*>(workspace);
  float* ws_s = reinterpret_cast<float*>(ws + L.o_s);
  void* ws_pe = ws + L.o_pe;
  float* ws_y = reinterpret_cast<float*>(ws + L.o_dq);
  const int f16 = d->dtype == FA_DTYPE_FP16;

  for (int64_t h0 = 0; h0 < L.heads; h0 += L.hc) {
    const int64_t hc = L.heads - h0 < L.hc ? L.heads - h0 : L.hc;
    ScoreArgs s{};
    s.q = e16(query, h0 * L.NMD);
    s.ws_s = ws_s;
    s.mask = atten_mask;
    s.head0 = (int32_t)h0;
    s.heads = (int32_t)hc;
    s.H = d->H;
    s.N = d->N;
    s.M = d->M;
    s.K = d->K;
    s.D = d->D;
    s.scale = d->scale_value;
    s.f16 = f16;
    s.x1 = e16(key1, h0 * L.NKD);
    s.by_m = 0;
    s.epi = 2;
    if (launch_scores(s, stream)) return FA_ERR_RUNTIME;
    s.x1 = e16(key2, h0 * L.KMD);
    s.by_m = 1;
    s.epi = 3;
    if (launch_scores(s, stream)) return FA_ERR_RUNTIME;

    SoftmaxArgs m{};
    m.ws_s = ws_s;
    m.p = ws_pe;
    m.smax = softmax_max + h0 * L.NM * 8;
    m.ssum = softmax_sum + h0 * L.NM * 8;
    m.mask = atten_mask;
    m.head0 = (int32_t)h0;
    m.heads = (int32_t)hc;
    m.H = d->H;
    m.N = d->N;
    m.M = d->M;
    m.K = d->K;
    m.scale = d->scale_value;
    m.f16 = f16;
    if (launch_softmax(m, stream)) return FA_ERR_RUNTIME;

    // Y = P V1 (batched over n, fp32) + P V2 (batched over m)
    GemmArgs a = gemm_base(d, hc);
    a.a_si = d->K; a.a_st = 1; a.a_sh = L.NMK; a.a_sz = L.MK; a.a_tc = 1;
    a.b_sj = 1; a.b_st = d->D; a.b_sh = L.NKD; a.b_sz = L.KD; a.b_tc = 0;
    a.c_si = d->D; a.c_sh = L.NMD; a.c_sz = L.MD;
    a.I = d->M; a.J = d->D; a.T = d->K; a.nb = d->N;
    a.a = ws_pe; a.b = e16(value1, h0 * L.NKD); a.c = ws_y; a.out_f32 = 1; a.alpha = 1.f;
    if (launch_gemm(a, stream)) return FA_ERR_RUNTIME;
    GemmArgs b = gemm_base(d, hc);
    b.a_si = L.MK; b.a_st = 1; b.a_sh = L.NMK; b.a_sz = d->K; b.a_tc = 1;
    b.b_sj = 1; b.b_st = L.MD; b.b_sh = L.KMD; b.b_sz = d->D; b.b_tc = 0;
    b.c_si = L.MD; b.c_sh = L.NMD; b.c_sz = d->D;
    b.I = d->N; b.J = d->D; b.T = d->K; b.nb = d->M;
    b.a = ws_pe; b.b = e16(value2, h0 * L.KMD); b.c = e16(attention_out, h0 * L.NMD); b.addend = ws_y;
    b.alpha = 1.f;
    if (launch_gemm(b, stream)) return FA_ERR_RUNTIME;
  }
  return FA_OK;
}

}  // extern "C"
