// C-ABI layer of la_gdn: argument validation, workspace carving, per-kernel
// timing hooks.  Every check here runs before any HIP call, so a rejected call
// touches neither the device nor any output.
//
// The validation rules mirror the cuDNN "Linear Attention" page ("Layout":
// rank-3 THD views with a contiguous innermost axis; "Engines": unsupported
// head dims are declined with an error) and the alignment contract of the
// 128-bit loads named in the cudnn-frontend PR "Further reduce FROST LA CPU
// overhead + fully support all L2norm, beta, gate fusion" (review of the state
// downcast and l2norm launchers: 16-byte base pointers, outer strides that keep
// 16-byte alignment).

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "la_gdn.h"
#include "la_gdn_internal.h"

namespace {

thread_local std::string g_error;

la_status fail(la_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_error = buf;
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The kernels address the rows of one chunk (and the 4-byte rows of g and beta) from the
// chunk's first row with 32-bit byte offsets: 66 rows of a 16-bit tensor, or 64 of a
// 32-bit one, at a token stride below 2^24 elements stay below 2^32 bytes.
constexpr int64_t kMaxTokenStride = int64_t(1) << 24;

int64_t round8(int64_t x) { return (x + 7) & ~int64_t(7); }

// Descriptor checks shared by both calls and by the workspace query.
la_status check_desc(const la_gdn_desc *d)
{
    if (!d) return fail(LA_ERR_INVALID_ARGUMENT, "desc is NULL");
    if (d->num_seqs < 0) return fail(LA_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0, got %d", d->num_seqs);
    if (d->total_tokens < 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "total_tokens must be >= 0, got %lld", (long long)d->total_tokens);
    if (d->total_tokens > INT32_MAX - 64)
        return fail(LA_ERR_UNSUPPORTED, "total_tokens %lld exceeds the int32 token index range",
                    (long long)d->total_tokens);
    if (d->num_qk_heads < 1) return fail(LA_ERR_INVALID_ARGUMENT, "num_qk_heads must be >= 1, got %d", d->num_qk_heads);
    if (d->num_v_heads < 1) return fail(LA_ERR_INVALID_ARGUMENT, "num_v_heads must be >= 1, got %d", d->num_v_heads);
    if (d->num_v_heads % d->num_qk_heads != 0)
        return fail(LA_ERR_UNSUPPORTED, "num_v_heads (%d) must be a multiple of num_qk_heads (%d)",
                    d->num_v_heads, d->num_qk_heads);
    if (d->head_dim_k != 64 && d->head_dim_k != 128)
        return fail(LA_ERR_UNSUPPORTED, "head_dim_k must be 64 or 128, got %d", d->head_dim_k);
    if (d->head_dim_v != 64 && d->head_dim_v != 128)
        return fail(LA_ERR_UNSUPPORTED, "head_dim_v must be 64 or 128, got %d", d->head_dim_v);
    const int64_t max_chunks = (d->total_tokens + 63) / 64 + d->num_seqs;
    if (max_chunks > INT32_MAX / 2)
        return fail(LA_ERR_UNSUPPORTED, "too many chunks (%lld)", (long long)max_chunks);
    const int64_t units = (int64_t)d->num_seqs * d->num_v_heads * 16;
    if (units > INT32_MAX)
        return fail(LA_ERR_UNSUPPORTED, "num_seqs * num_v_heads too large (%lld)", (long long)units / 16);
    return LA_OK;
}

// A bf16 [T, heads, dim] operand: 16-byte base, unit innermost stride (implied),
// outer strides multiples of 8 elements and large enough not to overlap rows.
la_status check_thd(const char *name, const void *ptr, int64_t st_t, int64_t st_h, int heads, int dim,
                    int64_t T, bool offsets32 = true)
{
    if (!ptr) return fail(LA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned16(ptr)) return fail(LA_ERR_INVALID_ARGUMENT, "%s base pointer is not 16-byte aligned", name);
    if (st_h % 8 != 0 || st_t % 8 != 0)
        return fail(LA_ERR_INVALID_ARGUMENT,
                    "%s strides (t=%lld, h=%lld) must be multiples of 8 elements (16 bytes)", name,
                    (long long)st_t, (long long)st_h);
    if (heads > 1 && st_h < dim)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s head stride %lld is smaller than the head dim %d", name,
                    (long long)st_h, dim);
    if (T > 1 && st_t < (int64_t)(heads - 1) * st_h + dim)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s token stride %lld overlaps its heads", name, (long long)st_t);
    if (offsets32 && T > 1 && st_t >= kMaxTokenStride)
        return fail(LA_ERR_UNSUPPORTED,
                    "%s token stride %lld: strides of 2^24 elements or more are not supported (the kernels "
                    "address the rows of a chunk with 32-bit byte offsets)", name, (long long)st_t);
    return LA_OK;
}

la_status check_rows(const char *name, const void *ptr, int64_t st_t, int heads, int64_t T)
{
    if (!ptr) return fail(LA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
    if (!aligned4(ptr)) return fail(LA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
    if (T > 1 && st_t < heads)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s token stride %lld is smaller than num_v_heads %d", name,
                    (long long)st_t, heads);
    if (T > 1 && st_t >= kMaxTokenStride)
        return fail(LA_ERR_UNSUPPORTED,
                    "%s token stride %lld: strides of 2^24 elements or more are not supported (the kernels "
                    "address the rows of a chunk with 32-bit byte offsets)", name, (long long)st_t);
    return LA_OK;
}

la_status check_f32(const char *name, const void *ptr, bool required)
{
    if (!ptr) return required ? fail(LA_ERR_INVALID_ARGUMENT, "%s is NULL", name) : LA_OK;
    if (!aligned4(ptr)) return fail(LA_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
    return LA_OK;
}

int householder(const la_gdn_options *f);
bool token_major(const la_gdn_options *f);

// beta (fp32, or bf16 logits under the in-kernel sigmoid) and the safe-gate parameters.
la_status check_beta_and_fusion(const void *beta, const la_gdn_desc &d, const la_gdn_options *f)
{
    const int64_t T = d.total_tokens;
    const bool logits = f && f->beta_sigmoid;
    if (!beta) return fail(LA_ERR_INVALID_ARGUMENT, "beta is NULL");
    if (logits ? (reinterpret_cast<uintptr_t>(beta) & 1u) != 0 : !aligned4(beta))
        return fail(LA_ERR_INVALID_ARGUMENT, "beta is not %d-byte aligned", logits ? 2 : 4);
    if (T > 1 && !token_major(f) && d.beta_stride_t < d.num_v_heads)
        return fail(LA_ERR_INVALID_ARGUMENT, "beta token stride %lld is smaller than num_v_heads %d",
                    (long long)d.beta_stride_t, d.num_v_heads);
    if (T > 1 && !token_major(f) && d.beta_stride_t >= kMaxTokenStride)
        return fail(LA_ERR_UNSUPPORTED,
                    "beta token stride %lld: strides of 2^24 elements or more are not supported (the kernels "
                    "address the rows of a chunk with 32-bit byte offsets)", (long long)d.beta_stride_t);
    if (!f) return LA_OK;
    if (f->dt_bias && !f->a_log) return fail(LA_ERR_INVALID_ARGUMENT, "dt_bias is given without a_log");
    la_status st = check_f32("a_log", f->a_log, false);
    if (st == LA_OK) st = check_f32("dt_bias", f->dt_bias, false);
    return st;
}

int householder(const la_gdn_options *f) { return f && f->num_householder > 1 ? f->num_householder : 1; }

// Gated Delta Product: n update rows per token, within the int32 row range.
la_status check_householder(const la_gdn_desc &d, const la_gdn_options *f)
{
    if (!f) return LA_OK;
    if (f->num_householder < 0 || f->num_householder > 64)
        return fail(LA_ERR_UNSUPPORTED, "num_householder must be in 0..64, got %d", f->num_householder);
    const int64_t rows = d.total_tokens * householder(f);
    if (rows > INT32_MAX - 64 || (rows + 63) / 64 + d.num_seqs > INT32_MAX / 2)
        return fail(LA_ERR_UNSUPPORTED, "total_tokens * num_householder (%lld) exceeds the int32 row range",
                    (long long)rows);
    if (householder(f) > 1 && f->checkpoint_every_n_tokens != 0)
        return fail(LA_ERR_UNSUPPORTED, "the state series is not available with num_householder > 1");
    return LA_OK;
}

bool token_major(const la_gdn_options *f) { return householder(f) > 1 && f->householder_token_major != 0; }

// Gated Delta Product, token-major operands ("Linear Attention" page, its description of
// GDP): n update rows of `heads` x `dim` per token, su apart, the tokens st apart.
la_status check_update_rows(const char *name, int64_t st, int64_t su, int64_t row_extent, int n, int64_t T,
                            bool vec16)
{
    if (vec16 && su % 8 != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s update stride %lld must be a multiple of 8 elements (16 bytes)",
                    name, (long long)su);
    if (su < row_extent)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s update stride %lld overlaps its heads", name, (long long)su);
    if (T > 1 && st < (int64_t)(n - 1) * su + row_extent)
        return fail(LA_ERR_INVALID_ARGUMENT, "%s token stride %lld overlaps its %d update rows", name,
                    (long long)st, n);
    if (st >= (1 << 23) || su >= (1 << 23))
        return fail(LA_ERR_UNSUPPORTED, "%s strides of 2^23 elements or more are not supported", name);
    return LA_OK;
}

// The kernels address a chunk's update rows with 32-bit offsets from its first token:
// 64 token strides plus 64 update strides stay below 2^30 elements.
la_status check_update_major_range(const char *name, int64_t row_stride, int n)
{
    if (n > 1 && row_stride * n >= (1 << 23))
        return fail(LA_ERR_UNSUPPORTED, "%s: row stride * num_householder of 2^23 elements or more is not supported",
                    name);
    return LA_OK;
}

// k, v and beta of either layout; `TU` = update rows.
la_status check_kvb(const la_gdn_desc &d, const void *k, const void *v, const la_gdn_options *f)
{
    const int64_t T = d.total_tokens;
    la_status st;
    if (!token_major(f)) {
        const int64_t TU = T * householder(f);   // update rows of k, v and beta
        if ((st = check_thd("k", k, d.k_stride_t, d.k_stride_h, d.num_qk_heads, d.head_dim_k, TU)) != LA_OK)
            return st;
        if ((st = check_thd("v", v, d.v_stride_t, d.v_stride_h, d.num_v_heads, d.head_dim_v, TU)) != LA_OK)
            return st;
        const int n = householder(f);
        if ((st = check_update_major_range("k", d.k_stride_t, n)) != LA_OK) return st;
        if ((st = check_update_major_range("v", d.v_stride_t, n)) != LA_OK) return st;
        return check_update_major_range("beta", d.beta_stride_t, n);
    }
    const int n = householder(f);
    // pointers and the head strides as for one row, then the update and token strides
    if ((st = check_thd("k", k, d.k_stride_t, d.k_stride_h, d.num_qk_heads, d.head_dim_k, 1)) != LA_OK) return st;
    if ((st = check_thd("v", v, d.v_stride_t, d.v_stride_h, d.num_v_heads, d.head_dim_v, 1)) != LA_OK) return st;
    if ((st = check_update_rows("k", d.k_stride_t, f->k_stride_update,
                                (int64_t)(d.num_qk_heads - 1) * d.k_stride_h + d.head_dim_k, n, T, true)) != LA_OK)
        return st;
    if ((st = check_update_rows("v", d.v_stride_t, f->v_stride_update,
                                (int64_t)(d.num_v_heads - 1) * d.v_stride_h + d.head_dim_v, n, T, true)) != LA_OK)
        return st;
    return check_update_rows("beta", d.beta_stride_t, f->beta_stride_update, d.num_v_heads, n, T, false);
}

// Row strides of k, v and beta as the kernels take them: for n > 1, token strides plus the
// stride between the updates of one token.
void set_update_strides(la::Prob &p, const la_gdn_options *f)
{
    p.kstu = p.kst;
    p.vstu = p.vst;
    p.bstu = p.bst;
    if (p.nh == 1) return;
    if (token_major(f)) {
        p.kstu = f->k_stride_update;
        p.vstu = f->v_stride_update;
        p.bstu = f->beta_stride_update;
    } else {
        p.kst *= p.nh;
        p.vst *= p.nh;
        p.bst *= p.nh;
    }
}

// The state series options ("Linear Attention" page, "States and checkpoints").
la_status check_checkpoints(const la_gdn_options *f, bool summary)
{
    if (!f || f->checkpoint_every_n_tokens == 0) return LA_OK;
    if (summary) return fail(LA_ERR_UNSUPPORTED, "the summary returns no state series (checkpoint_every_n_tokens)");
    const int n = f->checkpoint_every_n_tokens;
    if (n < 0) return fail(LA_ERR_INVALID_ARGUMENT, "checkpoint_every_n_tokens must be >= 0, got %d", n);
    if (n % 64 != 0)
        return fail(LA_ERR_UNSUPPORTED, "checkpoint_every_n_tokens must be a multiple of the 64-token chunk, got %d",
                    n);
    if (f->checkpoint_capacity < 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "checkpoint_capacity must be >= 0");
    if (f->checkpoint_capacity > 0 && !f->checkpoints)
        return fail(LA_ERR_INVALID_ARGUMENT, "checkpoints is NULL");
    const uintptr_t a = reinterpret_cast<uintptr_t>(f->checkpoints);
    if ((a & (f->checkpoint_fp32 ? 3u : 1u)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "checkpoints is not %d-byte aligned", f->checkpoint_fp32 ? 4 : 2);
    return LA_OK;
}

// With one token (one update row) a tensor's token stride is never used to reach a second
// row, and the argument checks accept any value for it (a broadcast view has 0).  The
// kernels size each chunk's buffer range as rows x token stride, so such a stride would
// read the row as zeros: it is replaced by the row's own extent, which gives the same
// addresses for the one row and puts every padding row past the range.  Runs after
// set_update_strides (update-row strides of the Gated Delta Product).
void normalize_single_token(la::Prob &p, const la_gdn_options *f)
{
    if (p.T != 1) return;
    p.qst = round8((int64_t)(p.HK - 1) * p.qsh + p.K);
    p.ost = round8((int64_t)(p.HV - 1) * p.osh + p.V);
    p.gst = p.HV;
    const int64_t ek = round8((int64_t)(p.HK - 1) * p.ksh + p.K);
    const int64_t ev = round8((int64_t)(p.HV - 1) * p.vsh + p.V);
    if (p.nh == 1) {
        p.kst = p.kstu = ek;
        p.vst = p.vstu = ev;
        p.bst = p.bstu = p.HV;
    } else if (token_major(f)) {
        // one token: its update rows are kstu apart; a token stride of n update strides
        // puts every row of a following (absent) token past the range
        p.kst = p.nh * p.kstu;
        p.vst = p.nh * p.vstu;
        p.bst = p.nh * p.bstu;
    }
}

void set_beta_and_fusion(la::Prob &p, const void *beta, const la_gdn_options *f)
{
    const bool logits = f && f->beta_sigmoid;
    p.beta = logits ? nullptr : static_cast<const float *>(beta);
    p.beta16 = logits ? static_cast<const __bf16 *>(beta) : nullptr;
    p.a_log = f ? f->a_log : nullptr;
    p.dt_bias = f ? f->dt_bias : nullptr;
    p.nh = householder(f);
    p.inv_nh = 1.0f / (float)p.nh;
    p.max_chunks = (int32_t)((p.T * p.nh + 63) / 64 + p.N);
    const bool series = f && f->checkpoint_every_n_tokens > 0 && f->checkpoint_capacity > 0;
    p.ck_every = series ? f->checkpoint_every_n_tokens : 0;
    p.ck_fp32 = series && f->checkpoint_fp32 ? 1 : 0;
    p.ck = series ? f->checkpoints : nullptr;
    p.ck_cap = series ? f->checkpoint_capacity : 0;
}

// ---------------------------------------------------------------------------
// per-kernel timing

struct Profiler {
    std::mutex mu;
    bool enabled = false;
    struct Pending {
        int id;
        hipEvent_t a, b;
    };
    std::vector<Pending> pending;
    std::vector<hipEvent_t> free_events;
    hipEvent_t open[LA_KERNEL_COUNT] = {};
    double total_ms[LA_KERNEL_COUNT] = {};
    int64_t launches[LA_KERNEL_COUNT] = {};
    hipError_t err = hipSuccess;

    hipEvent_t get()
    {
        if (!free_events.empty()) {
            hipEvent_t e = free_events.back();
            free_events.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) err = r;
        return e;
    }
};

Profiler &profiler()
{
    static Profiler p;
    return p;
}

void prof_before(int id, hipStream_t s, void *)
{
    Profiler &P = profiler();
    std::lock_guard<std::mutex> g(P.mu);
    hipEvent_t e = P.get();
    if (!e) return;
    const hipError_t r = hipEventRecord(e, s);
    if (r != hipSuccess) P.err = r;
    P.open[id] = e;
}

void prof_after(int id, hipStream_t s, void *)
{
    Profiler &P = profiler();
    std::lock_guard<std::mutex> g(P.mu);
    if (!P.open[id]) return;
    hipEvent_t e = P.get();
    if (!e) return;
    const hipError_t r = hipEventRecord(e, s);
    if (r != hipSuccess) P.err = r;
    P.pending.push_back({id, P.open[id], e});
    P.open[id] = nullptr;
}

const la::LaunchHook *current_hook()
{
    static const la::LaunchHook hook = {prof_before, prof_after, nullptr};
    Profiler &P = profiler();
    std::lock_guard<std::mutex> g(P.mu);
    return P.enabled ? &hook : nullptr;
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cu_count()
{
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

la::Prob make_prob(const la_gdn_desc *d, int l2norm)
{
    la::Prob p{};
    p.N = d->num_seqs;
    p.T = d->total_tokens;
    p.HK = d->num_qk_heads;
    p.HV = d->num_v_heads;
    p.K = d->head_dim_k;
    p.V = d->head_dim_v;
    p.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim_k);
    p.l2norm = l2norm ? 1 : 0;
    p.nh = 1;
    p.max_chunks = (int32_t)((d->total_tokens + 63) / 64 + d->num_seqs);
    p.intra_grid = 3 * device_cu_count();
    {
        // The operands the intra pass hands to the inter pass (-W, U~, P^T, scalars per
        // (chunk, value head)): while they fit in about half of the 256 MiB Infinity Cache
        // the inter pass reads them from there; beyond that, non-temporal stores keep them
        // from displacing the cache's other lines and measured faster (k_inter at 8 x 4096
        // tokens, HV = 16: 229 -> 207 us; at 4096 tokens: 34.7 -> 38.0 us the other way).
        const int64_t per_item = 64 * (int64_t)(d->head_dim_k + d->head_dim_v) * 2 + 7 * la::kFrag;
        const int64_t ops = (int64_t)p.max_chunks * d->num_v_heads * per_item;
        p.stream_ops = ops > ((int64_t)128 << 20) ? 1 : 0;
    }
    p.qst = d->q_stride_t;
    p.qsh = d->q_stride_h;
    p.kst = d->k_stride_t;
    p.ksh = d->k_stride_h;
    p.vst = d->v_stride_t;
    p.vsh = d->v_stride_h;
    p.ost = d->o_stride_t;
    p.osh = d->o_stride_h;
    p.gst = d->g_stride_t;
    p.bst = d->beta_stride_t;
    return p;
}

// cu64: cu_seqlens given as int64 (p.cu is then replaced by the workspace's int32 copy).
la_status launch(la::Prob p, void *workspace, size_t workspace_bytes, bool summary, hipStream_t stream,
                 const int64_t *cu64 = nullptr)
{
    const la::WsLayout L = la::workspace_layout(p.N, p.T * p.nh, p.HK, p.HV, p.K, p.V, summary);
    if (p.N == 0) return LA_OK;  // nothing to compute and nothing to write
    if (!workspace) return fail(LA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(LA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
    const la::Ws w = la::carve_workspace(workspace, L, summary);
    const la::LaunchHook *hook = current_hook();
    if (cu64) {
        if (hook) hook->before(LA_KERNEL_SCHED, stream, hook->ctx);
        const hipError_t ec = la::convert_cu64(cu64, w.cu32, p.N + 1, stream);
        if (hook) hook->after(LA_KERNEL_SCHED, stream, hook->ctx);
        if (ec != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(ec));
        p.cu = w.cu32;
    }
    const hipError_t e = la::run_pipeline(p, w, summary, stream, hook);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

}  // namespace

namespace la {

la_status fail_message(la_status st, const char *msg) { return fail(st, "%s", msg); }

WsLayout workspace_layout(int64_t N, int64_t T, int64_t HK, int64_t HV, int64_t K, int64_t V, bool summary,
                          int bwd)
{
    (void)HK;
    WsLayout L{};
    const bool fwd_ops = bwd != 1;          // the forward's operands (forward, summary, full backward)
    const int64_t C = (T + 63) / 64 + N;   // chunk ids
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.hdr = take(256);
    L.seq_info = take(sizeof(int4) * (size_t)N);
    L.chunks = take(sizeof(int4) * (size_t)C);
    L.order = take(sizeof(int32_t) * (size_t)N);
    const size_t items = (size_t)(C * HV);
    L.WF = take(fwd_ops ? items * 64 * K * 2 : 0);        // 64 x K bf16
    L.PF = take(summary || !fwd_ops ? 0 : items * 6 * la::kFrag);
    L.UH = take(fwd_ops ? items * 64 * V * 2 : 0);        // 64 x V fp16
    L.SC = take(items * la::kScalars * 4);
    L.cu32 = take(sizeof(int32_t) * (size_t)(N + 1));
    L.WTF = take(bwd ? items * 64 * K * 2 : 0);
    L.PTF = take(bwd ? items * 6 * la::kFrag : 0);
    L.TB = take(bwd == 2 ? items * 64 * 64 * 2 : 0);
    L.SB = take(bwd == 2 ? items * la::kScalars * 4 : 0);
    L.CK = take(bwd == 2 ? items * K * V * 4 : 0);
    L.DSN = take(bwd == 2 ? items * K * V * 4 : 0);
    L.DU = take(bwd == 2 ? items * 64 * V * 2 : 0);
    // per-value-head q and k gradients, summed over each head group afterwards (with one
    // value head per q/k head the intra pass writes dq and dk itself)
    const bool qk_sums = bwd == 2 && HV != HK;
    L.DQH = take(qk_sums ? (size_t)T * HV * K * 4 : 0);
    L.DKH = take(qk_sums ? (size_t)T * HV * K * 4 : 0);
    L.total = off;
    return L;
}

Ws carve_workspace(void *base, const WsLayout &L, bool summary)
{
    char *b = static_cast<char *>(base);
    Ws w{};
    w.hdr = reinterpret_cast<int32_t *>(b + L.hdr);
    w.seq_info = reinterpret_cast<int4 *>(b + L.seq_info);
    w.chunks = reinterpret_cast<int4 *>(b + L.chunks);
    w.order = reinterpret_cast<int32_t *>(b + L.order);
    w.WF = reinterpret_cast<uint4 *>(b + L.WF);
    w.PF = summary ? nullptr : reinterpret_cast<uint4 *>(b + L.PF);
    w.UH = reinterpret_cast<uint2 *>(b + L.UH);
    w.SC = reinterpret_cast<float *>(b + L.SC);
    w.cu32 = reinterpret_cast<int32_t *>(b + L.cu32);
    w.WTF = reinterpret_cast<uint4 *>(b + L.WTF);
    w.PTF = reinterpret_cast<uint4 *>(b + L.PTF);
    w.TB = reinterpret_cast<uint4 *>(b + L.TB);
    w.SB = reinterpret_cast<float *>(b + L.SB);
    w.CK = reinterpret_cast<float *>(b + L.CK);
    w.DSN = reinterpret_cast<float *>(b + L.DSN);
    w.DU = reinterpret_cast<__bf16 *>(b + L.DU);
    w.DQH = reinterpret_cast<float *>(b + L.DQH);
    w.DKH = reinterpret_cast<float *>(b + L.DKH);
    return w;
}

}  // namespace la

extern "C" {

size_t la_gdn_workspace_bytes(const la_gdn_desc *desc, int is_summary)
{
    if (check_desc(desc) != LA_OK) return 0;
    return la::workspace_layout(desc->num_seqs, desc->total_tokens, desc->num_qk_heads, desc->num_v_heads,
                                desc->head_dim_k, desc->head_dim_v, is_summary != 0)
        .total;
}

size_t la_gdn_workspace_bytes_ex(const la_gdn_desc *desc, int is_summary, const la_gdn_options *options)
{
    if (check_desc(desc) != LA_OK || check_householder(*desc, options) != LA_OK) return 0;
    return la::workspace_layout(desc->num_seqs, desc->total_tokens * householder(options), desc->num_qk_heads,
                                desc->num_v_heads, desc->head_dim_k, desc->head_dim_v, is_summary != 0)
        .total;
}

la_status la_gdn_fwd(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const float *initial_state, void *out,
                     float *final_state, int l2norm, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return la_gdn_fwd_ex(desc, q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, l2norm, nullptr,
                            workspace, workspace_bytes, stream);
}

la_status la_gdn_fwd_ex(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                           const void *beta, const void *cu_seqlens, const float *initial_state, void *out,
                           float *final_state, int l2norm, const la_gdn_options *fusion, void *workspace,
                           size_t workspace_bytes, hipStream_t stream)
{
    g_error.clear();
    la_status st = check_desc(desc);
    if (st != LA_OK) return st;
    const la_gdn_desc &d = *desc;
    const int64_t T = d.total_tokens;
    if ((st = check_householder(d, fusion)) != LA_OK) return st;
    if ((st = check_thd("q", q, d.q_stride_t, d.q_stride_h, d.num_qk_heads, d.head_dim_k, T)) != LA_OK) return st;
    if ((st = check_kvb(d, k, v, fusion)) != LA_OK) return st;
    if ((st = check_thd("out", out, d.o_stride_t, d.o_stride_h, d.num_v_heads, d.head_dim_v, T, false)) != LA_OK)
        return st;
    if ((st = check_rows("g", g, d.g_stride_t, d.num_v_heads, T)) != LA_OK) return st;
    if ((st = check_beta_and_fusion(beta, d, fusion)) != LA_OK) return st;
    const bool cu64 = fusion && fusion->cu_seqlens_int64;
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & (cu64 ? 7u : 3u)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is not %d-byte aligned", cu64 ? 8 : 4);
    if ((st = check_f32("initial_state", initial_state, false)) != LA_OK) return st;
    if ((st = check_f32("final_state", final_state, false)) != LA_OK) return st;
    if ((st = check_checkpoints(fusion, false)) != LA_OK) return st;

    la::Prob p = make_prob(desc, l2norm);
    p.q = static_cast<const __bf16 *>(q);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.g = g;
    set_beta_and_fusion(p, beta, fusion);
    set_update_strides(p, fusion);
    normalize_single_token(p, fusion);
    p.cu = cu64 ? nullptr : static_cast<const int32_t *>(cu_seqlens);
    p.s0 = initial_state;
    p.o = static_cast<__bf16 *>(out);
    p.sT = final_state;
    p.trans = nullptr;
    return launch(p, workspace, workspace_bytes, false, stream,
                  cu64 ? static_cast<const int64_t *>(cu_seqlens) : nullptr);
}

la_status la_gdn_summary(const la_gdn_desc *desc, const void *k, const void *v, const float *g, const float *beta,
                         const int32_t *cu_seqlens, const float *start_state, float *end_state, float *transition,
                         int l2norm, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return la_gdn_summary_ex(desc, k, v, g, beta, cu_seqlens, start_state, end_state, transition, l2norm, nullptr,
                                workspace, workspace_bytes, stream);
}

la_status la_gdn_summary_ex(const la_gdn_desc *desc, const void *k, const void *v, const float *g,
                               const void *beta, const void *cu_seqlens, const float *start_state,
                               float *end_state, float *transition, int l2norm, const la_gdn_options *fusion,
                               void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_error.clear();
    la_status st = check_desc(desc);
    if (st != LA_OK) return st;
    const la_gdn_desc &d = *desc;
    const int64_t T = d.total_tokens;
    if ((st = check_householder(d, fusion)) != LA_OK) return st;
    if ((st = check_kvb(d, k, v, fusion)) != LA_OK) return st;
    if ((st = check_rows("g", g, d.g_stride_t, d.num_v_heads, T)) != LA_OK) return st;
    if ((st = check_beta_and_fusion(beta, d, fusion)) != LA_OK) return st;
    const bool cu64 = fusion && fusion->cu_seqlens_int64;
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & (cu64 ? 7u : 3u)) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is not %d-byte aligned", cu64 ? 8 : 4);
    if ((st = check_f32("start_state", start_state, false)) != LA_OK) return st;
    if ((st = check_f32("end_state", end_state, true)) != LA_OK) return st;
    if ((st = check_f32("transition", transition, true)) != LA_OK) return st;
    if ((st = check_checkpoints(fusion, true)) != LA_OK) return st;

    la::Prob p = make_prob(desc, l2norm);
    p.q = nullptr;
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.g = g;
    set_beta_and_fusion(p, beta, fusion);
    set_update_strides(p, fusion);
    normalize_single_token(p, fusion);
    p.cu = cu64 ? nullptr : static_cast<const int32_t *>(cu_seqlens);
    p.s0 = start_state;
    p.o = nullptr;
    p.sT = end_state;
    p.trans = transition;
    return launch(p, workspace, workspace_bytes, true, stream,
                  cu64 ? static_cast<const int64_t *>(cu_seqlens) : nullptr);
}

la_status la_gdn_summary_bwd(const la_gdn_desc *desc, const void *q, const void *k, const float *g,
                             const float *beta, const int32_t *cu_seqlens, const void *d_out,
                             const float *d_end_state, float *d_start_state, int l2norm, void *workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    g_error.clear();
    la_status st = check_desc(desc);
    if (st != LA_OK) return st;
    const la_gdn_desc &d = *desc;
    const int64_t T = d.total_tokens;
    if ((st = check_thd("q", q, d.q_stride_t, d.q_stride_h, d.num_qk_heads, d.head_dim_k, T)) != LA_OK) return st;
    if ((st = check_thd("k", k, d.k_stride_t, d.k_stride_h, d.num_qk_heads, d.head_dim_k, T)) != LA_OK) return st;
    if ((st = check_thd("d_out", d_out, d.o_stride_t, d.o_stride_h, d.num_v_heads, d.head_dim_v, T)) != LA_OK)
        return st;
    if ((st = check_rows("g", g, d.g_stride_t, d.num_v_heads, T)) != LA_OK) return st;
    if ((st = check_beta_and_fusion(beta, d, nullptr)) != LA_OK) return st;
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    if (!aligned4(cu_seqlens)) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    if ((st = check_f32("d_end_state", d_end_state, false)) != LA_OK) return st;
    if ((st = check_f32("d_start_state", d_start_state, true)) != LA_OK) return st;

    la::Prob p = make_prob(desc, l2norm);
    p.q = static_cast<const __bf16 *>(q);
    p.k = static_cast<const __bf16 *>(k);
    p.g = g;
    p.beta = beta;
    p.cu = cu_seqlens;
    normalize_single_token(p, nullptr);
    if (p.N == 0) return LA_OK;
    // the reverse pass's operands fit in the summary's workspace (the size the header names)
    const size_t have_min = la::workspace_layout(p.N, p.T, p.HK, p.HV, p.K, p.V, true).total;
    if (!workspace) return fail(LA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < have_min)
        return fail(LA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, have_min);
    const la::WsLayout L = la::workspace_layout(p.N, p.T, p.HK, p.HV, p.K, p.V, false, 1);
    const la::Ws w = la::carve_workspace(workspace, L, false);
    const hipError_t e = la::run_summary_bwd(p, w, static_cast<const __bf16 *>(d_out), d_end_state, d_start_state,
                                             stream, current_hook());
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

size_t la_gdn_bwd_workspace_bytes(const la_gdn_desc *desc)
{
    if (check_desc(desc) != LA_OK) return 0;
    return la::workspace_layout(desc->num_seqs, desc->total_tokens, desc->num_qk_heads, desc->num_v_heads,
                                desc->head_dim_k, desc->head_dim_v, false, 2)
        .total;
}

static la_status bwd_impl(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                          const float *chunk_states, const void *d_out, const float *d_final_state, float *dq,
                          float *dk, float *dv, float *dg, float *dbeta, float *d_initial_state, int l2norm,
                          void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    g_error.clear();
    la_status st = check_desc(desc);
    if (st != LA_OK) return st;
    const la_gdn_desc &d = *desc;
    const int64_t T = d.total_tokens;
    if ((st = check_thd("q", q, d.q_stride_t, d.q_stride_h, d.num_qk_heads, d.head_dim_k, T)) != LA_OK) return st;
    if ((st = check_kvb(d, k, v, nullptr)) != LA_OK) return st;
    if ((st = check_thd("d_out", d_out, d.o_stride_t, d.o_stride_h, d.num_v_heads, d.head_dim_v, T)) != LA_OK)
        return st;
    if ((st = check_rows("g", g, d.g_stride_t, d.num_v_heads, T)) != LA_OK) return st;
    if ((st = check_beta_and_fusion(beta, d, nullptr)) != LA_OK) return st;
    if (!cu_seqlens) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
    if (!aligned4(cu_seqlens)) return fail(LA_ERR_INVALID_ARGUMENT, "cu_seqlens is not 4-byte aligned");
    if ((st = check_f32("initial_state", initial_state, false)) != LA_OK) return st;
    if ((st = check_f32("d_final_state", d_final_state, false)) != LA_OK) return st;
    if (!dq) return fail(LA_ERR_INVALID_ARGUMENT, "dq is NULL");
    if (!dk) return fail(LA_ERR_INVALID_ARGUMENT, "dk is NULL");
    if (!aligned16(dq) || !aligned16(dk))
        return fail(LA_ERR_INVALID_ARGUMENT, "dq and dk must be 16-byte aligned (they are written with 128-bit stores)");
    if ((st = check_f32("dv", dv, true)) != LA_OK) return st;
    if ((st = check_f32("dg", dg, true)) != LA_OK) return st;
    if ((st = check_f32("dbeta", dbeta, true)) != LA_OK) return st;
    if ((st = check_f32("d_initial_state", d_initial_state, true)) != LA_OK) return st;
    if (chunk_states && !aligned16(chunk_states))
        return fail(LA_ERR_INVALID_ARGUMENT, "chunk_states must be 16-byte aligned (it is read with 128-bit loads)");

    la::Prob p = make_prob(desc, l2norm);
    p.q = static_cast<const __bf16 *>(q);
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.g = g;
    p.beta = beta;
    p.kstu = p.kst;
    p.vstu = p.vst;
    p.bstu = p.bst;
    p.inv_nh = 1.0f;
    p.cu = cu_seqlens;
    p.s0 = initial_state;
    normalize_single_token(p, nullptr);
    if (p.N == 0) return LA_OK;
    const la::WsLayout L = la::workspace_layout(p.N, p.T, p.HK, p.HV, p.K, p.V, false, 2);
    if (!workspace) return fail(LA_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(LA_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(LA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);
    const la::Ws w = la::carve_workspace(workspace, L, false);
    la::BwdArgs a{};
    a.d_out = static_cast<const __bf16 *>(d_out);
    a.d_final = d_final_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dg = dg;
    a.dbeta = dbeta;
    a.d_init = d_initial_state;
    a.chunk_states = chunk_states;
    const hipError_t e = la::run_backward(p, w, a, stream, current_hook());
    if (e != hipSuccess) return fail(LA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

la_status la_gdn_bwd(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                     const float *beta, const int32_t *cu_seqlens, const float *initial_state, const void *d_out,
                     const float *d_final_state, float *dq, float *dk, float *dv, float *dg, float *dbeta,
                     float *d_initial_state, int l2norm, void *workspace, size_t workspace_bytes,
                     hipStream_t stream)
{
    return bwd_impl(desc, q, k, v, g, beta, cu_seqlens, initial_state, nullptr, d_out, d_final_state, dq, dk, dv, dg,
                    dbeta, d_initial_state, l2norm, workspace, workspace_bytes, stream);
}

la_status la_gdn_bwd_ex(const la_gdn_desc *desc, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const int32_t *cu_seqlens, const float *initial_state,
                        const float *chunk_states, const void *d_out, const float *d_final_state, float *dq,
                        float *dk, float *dv, float *dg, float *dbeta, float *d_initial_state, int l2norm,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return bwd_impl(desc, q, k, v, g, beta, cu_seqlens, initial_state, chunk_states, d_out, d_final_state, dq, dk,
                    dv, dg, dbeta, d_initial_state, l2norm, workspace, workspace_bytes, stream);
}

int32_t la_gdn_device_status(const void *workspace, hipStream_t stream)
{
    if (!workspace) {
        fail(LA_ERR_INVALID_ARGUMENT, "workspace is NULL");
        return -1;
    }
    int32_t h = -1;
    hipError_t e = hipMemcpyAsync(&h, workspace, sizeof h, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) {
        fail(LA_ERR_HIP, "status read failed: %s", hipGetErrorString(e));
        return -1;
    }
    return h;
}

const char *la_last_error_message(void) { return g_error.c_str(); }

la_status la_gdn_profile_enable(int enable)
{
    Profiler &P = profiler();
    std::lock_guard<std::mutex> g(P.mu);
    for (auto &pd : P.pending) {
        P.free_events.push_back(pd.a);
        P.free_events.push_back(pd.b);
    }
    P.pending.clear();
    for (int i = 0; i < LA_KERNEL_COUNT; ++i) {
        P.total_ms[i] = 0.0;
        P.launches[i] = 0;
        P.open[i] = nullptr;
    }
    P.err = hipSuccess;
    P.enabled = enable != 0;
    return LA_OK;
}

la_status la_gdn_profile_read(int32_t kernel_id, double *total_ms, int64_t *launches)
{
    if (kernel_id < 0 || kernel_id >= LA_KERNEL_COUNT)
        return fail(LA_ERR_INVALID_ARGUMENT, "kernel_id %d out of range", kernel_id);
    if (!total_ms || !launches) return fail(LA_ERR_INVALID_ARGUMENT, "output pointer is NULL");
    Profiler &P = profiler();
    std::lock_guard<std::mutex> g(P.mu);
    for (auto &pd : P.pending) {
        hipError_t e = hipEventSynchronize(pd.b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, pd.a, pd.b);
        if (e != hipSuccess) return fail(LA_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
        P.total_ms[pd.id] += ms;
        P.launches[pd.id] += 1;
        P.free_events.push_back(pd.a);
        P.free_events.push_back(pd.b);
    }
    P.pending.clear();
    if (P.err != hipSuccess) return fail(LA_ERR_HIP, "event record failed: %s", hipGetErrorString(P.err));
    *total_ms = P.total_ms[kernel_id];
    *launches = P.launches[kernel_id];
    return LA_OK;
}

const char *la_gdn_kernel_name(int32_t kernel_id)
{
    static const char *names[LA_KERNEL_COUNT] = {"k_sched", "k_intra", "k_inter", "k_bwd_intra"};
    return (kernel_id >= 0 && kernel_id < LA_KERNEL_COUNT) ? names[kernel_id] : "";
}

}  // extern "C"
