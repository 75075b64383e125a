// Drives the C ABI of la_gdn_api.cpp, built for the CPU with the kernel launchers and the
// HIP runtime stubbed (hip_stubs.cpp), under AddressSanitizer and
// UndefinedBehaviorSanitizer: every argument check, the workspace carving, the single-token
// stride normalisation, the options, the summary's mirror, the status read and the
// profiler.  Buffers that stand in for device memory are host allocations that are never
// read by the host layer.  Exits non-zero on the first unexpected result.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "la_gdn.h"
#include "stub_record.h"

static int g_checks = 0;

#define CHECK(cond)                                                                          \
    do {                                                                                     \
        ++g_checks;                                                                          \
        if (!(cond)) {                                                                       \
            std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__,     \
                         __LINE__, #cond, la_last_error_message());                          \
            std::exit(1);                                                                    \
        }                                                                                    \
    } while (0)

namespace {

// A 256-byte aligned host buffer standing in for device memory.
struct Buf {
    void *p = nullptr;
    explicit Buf(size_t n) { p = std::aligned_alloc(256, (n + 255) & ~size_t(255)); std::memset(p, 0, n); }
    ~Buf() { std::free(p); }
    char *c() const { return static_cast<char *>(p); }
};

la_gdn_desc desc(int N, int64_t T, int HK = 2, int HV = 4, int K = 128, int V = 128)
{
    la_gdn_desc d{};
    d.num_seqs = N;
    d.total_tokens = T;
    d.num_qk_heads = HK;
    d.num_v_heads = HV;
    d.head_dim_k = K;
    d.head_dim_v = V;
    d.scale = 0.f;
    d.q_stride_t = HK * K;
    d.q_stride_h = K;
    d.k_stride_t = HK * K;
    d.k_stride_h = K;
    d.v_stride_t = HV * V;
    d.v_stride_h = V;
    d.o_stride_t = HV * V;
    d.o_stride_h = V;
    d.g_stride_t = HV;
    d.beta_stride_t = HV;
    return d;
}

struct Args {
    Buf q, k, v, g, b, cu, s0, o, fin, tr, ws;
    size_t wsb;
    Args(const la_gdn_desc &d, bool summary)
        : q(2 * (size_t)d.total_tokens * d.q_stride_t + 64), k(2 * (size_t)d.total_tokens * d.k_stride_t + 64),
          v(2 * (size_t)d.total_tokens * d.v_stride_t + 64), g(4 * (size_t)d.total_tokens * d.g_stride_t + 64),
          b(4 * (size_t)d.total_tokens * d.beta_stride_t + 64), cu(8 * (size_t)(d.num_seqs + 1)),
          s0(4 * (size_t)d.num_seqs * d.num_v_heads * d.head_dim_k * d.head_dim_v + 64),
          o(2 * (size_t)d.total_tokens * d.o_stride_t + 64),
          fin(4 * (size_t)d.num_seqs * d.num_v_heads * d.head_dim_k * d.head_dim_v + 64),
          tr(4 * (size_t)d.num_seqs * d.num_v_heads * d.head_dim_k * d.head_dim_k + 64),
          ws(la_gdn_workspace_bytes(&d, summary ? 1 : 0)), wsb(la_gdn_workspace_bytes(&d, summary ? 1 : 0))
    {
    }
};

la_status fwd(const la_gdn_desc &d, Args &a, const la_gdn_options *opt = nullptr)
{
    return la_gdn_fwd_ex(&d, a.q.p, a.k.p, a.v.p, static_cast<float *>(a.g.p), a.b.p, a.cu.p,
                         static_cast<float *>(a.s0.p), a.o.p, static_cast<float *>(a.fin.p), 1, opt, a.ws.p,
                         a.wsb, nullptr);
}

la_status summ(const la_gdn_desc &d, Args &a, const la_gdn_options *opt = nullptr)
{
    return la_gdn_summary_ex(&d, a.k.p, a.v.p, static_cast<float *>(a.g.p), a.b.p, a.cu.p,
                             static_cast<float *>(a.s0.p), static_cast<float *>(a.fin.p),
                             static_cast<float *>(a.tr.p), 1, opt, a.ws.p, a.wsb, nullptr);
}

void valid_calls()
{
    const la_gdn_desc d = desc(3, 4096, 16, 16);
    Args a(d, false);
    const int before = g_stub.pipeline_calls;
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, static_cast<float *>(a.g.p), static_cast<float *>(a.b.p),
                     static_cast<int32_t *>(a.cu.p), nullptr, a.o.p, static_cast<float *>(a.fin.p), 1, a.ws.p,
                     a.wsb, nullptr) == LA_OK);
    CHECK(g_stub.pipeline_calls == before + 1 && !g_stub.last_summary);
    CHECK(g_stub.last.max_chunks == 4096 / 64 + 3 && g_stub.last.nh == 1);
    CHECK(g_stub.last.scale > 0.0883f && g_stub.last.scale < 0.0884f);   // 128^-1/2
    // the carved regions lie inside the workspace
    const char *lo = a.ws.c(), *hi = a.ws.c() + a.wsb;
    const char *parts[] = {reinterpret_cast<const char *>(g_stub.last_ws.hdr),
                           reinterpret_cast<const char *>(g_stub.last_ws.WF),
                           reinterpret_cast<const char *>(g_stub.last_ws.UH),
                           reinterpret_cast<const char *>(g_stub.last_ws.SC),
                           reinterpret_cast<const char *>(g_stub.last_ws.cu32)};
    for (const char *p : parts) CHECK(p >= lo && p < hi);

    Args s(d, true);
    CHECK(summ(d, s) == LA_OK && g_stub.last_summary);

    // int64 offsets go through the conversion kernel first
    la_gdn_options o{};
    o.cu_seqlens_int64 = 1;
    const int c64 = g_stub.cu64_calls;
    CHECK(fwd(d, a, &o) == LA_OK && g_stub.cu64_calls == c64 + 1);
    o.cu_seqlens_int64 = 0;

    // the state series and the fused transforms
    Buf ck(4 * 70 * 16 * 128 * 128), alog(64), dtb(64);
    o.checkpoint_every_n_tokens = 64;
    o.checkpoint_fp32 = 1;
    o.checkpoints = ck.p;
    o.checkpoint_capacity = 70;
    o.beta_sigmoid = 1;
    o.a_log = static_cast<float *>(alog.p);
    o.dt_bias = static_cast<float *>(dtb.p);
    CHECK(fwd(d, a, &o) == LA_OK);
    CHECK(g_stub.last.ck_every == 64 && g_stub.last.ck_fp32 == 1 && g_stub.last.beta16 && !g_stub.last.beta);

    // N = 0 launches nothing
    const la_gdn_desc e = desc(0, 0);
    Args ea(e, false);
    const int c = g_stub.pipeline_calls;
    CHECK(fwd(e, ea) == LA_OK && g_stub.pipeline_calls == c);
}

void single_token_strides()
{
    la_gdn_desc d = desc(1, 1, 2, 4, 64, 128);
    d.q_stride_t = d.k_stride_t = d.v_stride_t = d.o_stride_t = d.g_stride_t = d.beta_stride_t = 0;
    Args a(desc(1, 1, 2, 4, 64, 128), false);
    CHECK(fwd(d, a) == LA_OK);
    const la::Prob &p = g_stub.last;
    CHECK(p.qst == 2 * 64 && p.kst == 2 * 64 && p.vst == 4 * 128 && p.ost == 4 * 128);
    CHECK(p.gst == 4 && p.bst == 4 && p.kstu == p.kst && p.vstu == p.vst && p.bstu == p.bst);
    // token-major Gated Delta Product with one token: the token stride becomes n update strides
    la_gdn_options o{};
    o.num_householder = 3;
    o.householder_token_major = 1;
    o.k_stride_update = 2 * 64;
    o.v_stride_update = 4 * 128;
    o.beta_stride_update = 4;
    Args big(desc(1, 3, 2, 4, 64, 128), false);
    big.wsb = la_gdn_workspace_bytes_ex(&d, 0, &o);
    Buf ws(big.wsb);
    std::swap(big.ws.p, ws.p);
    CHECK(fwd(d, big, &o) == LA_OK);
    CHECK(g_stub.last.kst == 3 * 2 * 64 && g_stub.last.vst == 3 * 4 * 128 && g_stub.last.bst == 3 * 4);
}

void declines()
{
    const la_gdn_desc base = desc(2, 100);
    Args a(base, false);
    auto bad_desc = [&](void (*edit)(la_gdn_desc &), la_status want) {
        la_gdn_desc d = base;
        edit(d);
        CHECK(fwd(d, a) == want && std::strlen(la_last_error_message()) > 0);
    };
    bad_desc([](la_gdn_desc &d) { d.head_dim_k = 96; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.head_dim_v = 256; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.num_v_heads = 3; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.num_qk_heads = 0; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.num_seqs = -1; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.total_tokens = -1; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.total_tokens = INT64_MAX; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.num_seqs = INT32_MAX; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.q_stride_t = 100; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.k_stride_h = 4; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.o_stride_t = 8; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.g_stride_t = 2; }, LA_ERR_INVALID_ARGUMENT);
    bad_desc([](la_gdn_desc &d) { d.k_stride_t = int64_t(1) << 24; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.q_stride_t = int64_t(1) << 40; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.v_stride_t = INT64_MAX & ~int64_t(7); }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.g_stride_t = int64_t(1) << 24; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.beta_stride_t = int64_t(1) << 30; }, LA_ERR_UNSUPPORTED);
    bad_desc([](la_gdn_desc &d) { d.q_stride_h = -8; }, LA_ERR_INVALID_ARGUMENT);

    // pointers, alignment, workspace
    const la_gdn_desc &d = base;
    CHECK(la_gdn_fwd(&d, nullptr, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, a.o.p,
                     nullptr, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.c() + 8, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr,
                     a.o.p, nullptr, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, (float *)(a.g.c() + 2), (float *)a.b.p, (int32_t *)a.cu.p, nullptr,
                     a.o.p, nullptr, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, nullptr, nullptr, a.o.p, nullptr, 1,
                     a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, a.o.p,
                     nullptr, 1, nullptr, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, a.o.p,
                     nullptr, 1, a.ws.c() + 128, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_fwd(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, a.o.p,
                     nullptr, 1, a.ws.p, a.wsb - 1, nullptr) == LA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(la_gdn_summary(&d, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, nullptr,
                         (float *)a.tr.p, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_summary(&d, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr,
                         (float *)a.fin.p, nullptr, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);

    // options
    la_gdn_options o{};
    o.dt_bias = static_cast<float *>(a.g.p);
    CHECK(fwd(d, a, &o) == LA_ERR_INVALID_ARGUMENT);
    o = la_gdn_options{};
    o.checkpoint_every_n_tokens = 100;
    CHECK(fwd(d, a, &o) == LA_ERR_UNSUPPORTED);
    o.checkpoint_every_n_tokens = 64;
    o.checkpoint_capacity = 5;
    CHECK(fwd(d, a, &o) == LA_ERR_INVALID_ARGUMENT);     // no buffer
    CHECK(summ(d, a, &o) == LA_ERR_UNSUPPORTED);         // no series from the summary
    o = la_gdn_options{};
    o.num_householder = 65;
    CHECK(fwd(d, a, &o) == LA_ERR_UNSUPPORTED);
    CHECK(la_gdn_workspace_bytes_ex(&d, 0, &o) == 0);
    o.num_householder = 2;
    o.checkpoint_every_n_tokens = 64;
    CHECK(fwd(d, a, &o) == LA_ERR_UNSUPPORTED);
    o = la_gdn_options{};
    o.num_householder = 2;
    o.householder_token_major = 1;
    o.k_stride_update = 2 * 128 + 4;
    CHECK(fwd(d, a, &o) == LA_ERR_INVALID_ARGUMENT);
    o.cu_seqlens_int64 = 1;
    CHECK(la_gdn_fwd_ex(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, a.b.p, a.cu.c() + 4, nullptr, a.o.p, nullptr, 1,
                        &o, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
}

void summary_bwd()
{
    const la_gdn_desc d = desc(2, 300, 2, 4, 64, 64);
    Args a(d, true);
    const int before = g_stub.sbwd_calls;
    CHECK(la_gdn_summary_bwd(&d, a.q.p, a.k.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, a.o.p, nullptr,
                             (float *)a.fin.p, 1, a.ws.p, a.wsb, nullptr) == LA_OK);
    CHECK(g_stub.sbwd_calls == before + 1);
    CHECK(la_gdn_summary_bwd(&d, a.q.p, a.k.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, a.o.p, nullptr,
                             nullptr, 1, a.ws.p, a.wsb, nullptr) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_summary_bwd(&d, a.q.p, a.k.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, a.o.p, nullptr,
                             (float *)a.fin.p, 1, a.ws.p, 64, nullptr) == LA_ERR_WORKSPACE_TOO_SMALL);
}

void full_backward()
{
    const la_gdn_desc d = desc(3, 700, 2, 4, 128, 64);
    Args a(d, false);
    const size_t wsb = la_gdn_bwd_workspace_bytes(&d);
    CHECK(wsb > a.wsb);
    Buf ws(wsb), dq(4 * 700 * 2 * 128), dk(4 * 700 * 2 * 128), dv(4 * 700 * 4 * 64), dg(4 * 700 * 4),
        db(4 * 700 * 4), di(4 * 3 * 4 * 128 * 64);
    auto call = [&](const void *dout, float *dqp, void *w, size_t n) {
        return la_gdn_bwd(&d, a.q.p, a.k.p, a.v.p, (float *)a.g.p, (float *)a.b.p, (int32_t *)a.cu.p, nullptr, dout,
                          nullptr, dqp, (float *)dk.p, (float *)dv.p, (float *)dg.p, (float *)db.p, (float *)di.p, 1, w,
                          n, nullptr);
    };
    const int before = g_stub.bwd_calls;
    CHECK(call(a.o.p, (float *)dq.p, ws.p, wsb) == LA_OK && g_stub.bwd_calls == before + 1);
    // every region of the backward's workspace lies inside it
    const char *lo = ws.c(), *hi = ws.c() + wsb;
    const char *parts[] = {reinterpret_cast<const char *>(g_stub.last_ws.WTF),
                           reinterpret_cast<const char *>(g_stub.last_ws.PTF),
                           reinterpret_cast<const char *>(g_stub.last_ws.TB),
                           reinterpret_cast<const char *>(g_stub.last_ws.SB),
                           reinterpret_cast<const char *>(g_stub.last_ws.CK),
                           reinterpret_cast<const char *>(g_stub.last_ws.DSN),
                           reinterpret_cast<const char *>(g_stub.last_ws.DU),
                           reinterpret_cast<const char *>(g_stub.last_ws.DQH),
                           reinterpret_cast<const char *>(g_stub.last_ws.DKH)};
    for (const char *p : parts) CHECK(p >= lo && p < hi);
    CHECK(call(nullptr, (float *)dq.p, ws.p, wsb) == LA_ERR_INVALID_ARGUMENT);
    CHECK(call(a.o.p, nullptr, ws.p, wsb) == LA_ERR_INVALID_ARGUMENT);
    CHECK(call(a.o.p, (float *)dq.p, ws.p, wsb - 1) == LA_ERR_WORKSPACE_TOO_SMALL);
    CHECK(call(a.o.p, (float *)dq.p, nullptr, wsb) == LA_ERR_INVALID_ARGUMENT);
}

void status_and_profiler()
{
    Buf ws(256);
    static_cast<int32_t *>(ws.p)[0] = LA_DEVICE_BAD_CU_SEQLENS;
    CHECK(la_gdn_device_status(ws.p, nullptr) == LA_DEVICE_BAD_CU_SEQLENS);
    CHECK(la_gdn_device_status(nullptr, nullptr) == -1);
    CHECK(la_gdn_profile_enable(1) == LA_OK);
    const la_gdn_desc d = desc(1, 64);
    Args a(d, false);
    for (int i = 0; i < 3; ++i) CHECK(fwd(d, a) == LA_OK);
    double ms = 0;
    int64_t n = 0;
    CHECK(la_gdn_profile_read(LA_KERNEL_INTRA, &ms, &n) == LA_OK && n == 3 && ms > 1.4 && ms < 1.6);
    CHECK(la_gdn_profile_read(LA_KERNEL_COUNT, &ms, &n) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_profile_read(LA_KERNEL_INTER, nullptr, &n) == LA_ERR_INVALID_ARGUMENT);
    CHECK(la_gdn_profile_enable(0) == LA_OK);
    CHECK(std::strcmp(la_gdn_kernel_name(LA_KERNEL_INTER), "k_inter") == 0);
    CHECK(std::strcmp(la_gdn_kernel_name(-1), "") == 0);
}

}  // namespace

int main()
{
    valid_calls();
    single_token_strides();
    declines();
    summary_bwd();
    full_backward();
    status_and_profiler();
    std::printf("abi_driver: %d checks passed\n", g_checks);
    return 0;
}
