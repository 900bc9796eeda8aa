// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation on
// the host, then the kernel launches on the caller's stream.  Every check runs
// before the first launch, so a rejected call launches nothing.

#include "kda.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda_launch.h"

namespace {

thread_local char g_err[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kda_status ok() {
    g_err[0] = '\0';
    return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A tensor read or written with vector accesses: non-NULL and 16-byte aligned.
kda_status need_vec(const void* p, const char* name) {
    if (!p) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return KDA_OK;
}

// An index array: non-NULL and naturally aligned.
kda_status need_idx(const void* p, size_t align, const char* name) {
    if (!p) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(KDA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return KDA_OK;
}

#define KDA_TRY(expr)                      \
    do {                                   \
        kda_status st_ = (expr);           \
        if (st_ != KDA_OK) return st_;     \
    } while (0)

kda_status check_cfg(const kda_config* c) {
    if (!c) return fail(KDA_ERR_INVALID_ARG, "cfg is NULL");
    if (c->num_heads < 1) return fail(KDA_ERR_INVALID_ARG, "num_heads must be >= 1 (got %d)", c->num_heads);
    if (c->head_k < 1 || c->head_v < 1)
        return fail(KDA_ERR_INVALID_ARG, "head_k and head_v must be >= 1 (got %d, %d)", c->head_k, c->head_v);
    if (c->act_dtype != KDA_F32 && c->act_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARG, "act_dtype must be KDA_F32 or KDA_BF16 (got %d)", c->act_dtype);
    if (c->state_dtype != KDA_F32 && c->state_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARG, "state_dtype must be KDA_F32 or KDA_BF16 (got %d)", c->state_dtype);
    if (!(std::isfinite(c->l2_eps) && c->l2_eps >= 0.f && std::isfinite(c->rms_eps) && c->rms_eps >= 0.f))
        return fail(KDA_ERR_INVALID_ARG, "l2_eps and rms_eps must be finite and >= 0");
    if (c->conv_width != 4)
        return fail(KDA_ERR_UNSUPPORTED, "conv_width must be 4 (got %d)", c->conv_width);
    if (c->head_k != c->head_v || (c->head_k != 32 && c->head_k != 64 && c->head_k != 128))
        return fail(KDA_ERR_UNSUPPORTED, "supported head sizes: dk == dv in {32, 64, 128} (got dk=%d dv=%d)",
                    c->head_k, c->head_v);
    return KDA_OK;
}

int act_bytes(const kda_config* c) { return c->act_dtype == KDA_BF16 ? 2 : 4; }

kda_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

kda_status check_copy_args(const kda_config* cfg, int32_t n, const void* src_state, const void* src_conv,
                           int32_t src_slots, const int32_t* src_idx, void* dst_state, void* dst_conv,
                           int32_t dst_slots, const int32_t* dst_idx) {
    KDA_TRY(check_cfg(cfg));
    if (n < 0) return fail(KDA_ERR_INVALID_ARG, "n must be >= 0 (got %d)", n);
    if (src_slots < 1 || dst_slots < 1) return fail(KDA_ERR_INVALID_ARG, "pool sizes must be >= 1");
    if (n == 0) return KDA_OK;
    // one workgroup per 4 KiB of each (pair, head)'s state and conv state
    const int64_t sb = static_cast<int64_t>(cfg->head_k) * cfg->head_v * (cfg->state_dtype == KDA_BF16 ? 2 : 4);
    const int64_t cb = static_cast<int64_t>(2 * cfg->head_k + cfg->head_v) * 3 * act_bytes(cfg);
    if (static_cast<int64_t>(n) * cfg->num_heads * ((sb + 4095) / 4096 + (cb + 4095) / 4096) > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "n * num_heads exceeds the launch grid");
    KDA_TRY(need_vec(src_state, "source state"));
    KDA_TRY(need_vec(src_conv, "source conv state"));
    KDA_TRY(need_vec(dst_state, "destination state"));
    KDA_TRY(need_vec(dst_conv, "destination conv state"));
    KDA_TRY(need_idx(src_idx, 4, "source ids"));
    KDA_TRY(need_idx(dst_idx, 4, "destination ids"));
    return KDA_OK;
}

kda::CopyParams copy_params(const kda_config* cfg, int32_t n, const void* src_state, const void* src_conv,
                            int32_t src_slots, const int32_t* src_idx, void* dst_state, void* dst_conv,
                            int32_t dst_slots, const int32_t* dst_idx) {
    kda::CopyParams p;
    p.n = n;
    p.H = cfg->num_heads;
    p.state_bytes = static_cast<int64_t>(cfg->head_k) * cfg->head_v * (cfg->state_dtype == KDA_BF16 ? 2 : 4);
    p.conv_bytes = static_cast<int64_t>(2 * cfg->head_k + cfg->head_v) * 3 * act_bytes(cfg);
    p.src_state = src_state;
    p.src_conv = src_conv;
    p.src_slots = src_slots;
    p.src_idx = src_idx;
    p.dst_state = dst_state;
    p.dst_conv = dst_conv;
    p.dst_slots = dst_slots;
    p.dst_idx = dst_idx;
    return p;
}

}  // namespace

int kda::set_error(int st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

extern "C" {

const char* kda_last_error(void) { return g_err; }

int64_t kda_num_checkpoints(int64_t start, int64_t len, int32_t interval) {
    if (interval <= 0 || len <= 0 || start < 0) return 0;
    const int64_t end = start + len;
    // multiples of interval in (start, end): floor((end-1)/N) - floor(start/N)
    return (end - 1) / interval - start / interval + 1;
}

namespace {

kda_status decode_common(const kda_config* cfg, int32_t B, int32_t T, const void* q, const void* k, const void* v,
                         const void* z, const float* g, const float* beta, const float* conv_w,
                         const float* norm_w, void* state_pool, void* conv_pool, int32_t num_slots,
                         const int32_t* slot, void* out, void* token_state, void* token_conv, void* stream) {
    KDA_TRY(check_cfg(cfg));
    if (B < 0) return fail(KDA_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (T < 1) return fail(KDA_ERR_INVALID_ARG, "T must be >= 1 (got %d)", T);
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1 (got %d)", num_slots);
    if (B == 0) return ok();
    if (static_cast<int64_t>(B) * cfg->num_heads > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "B * num_heads exceeds the launch grid");
    if (static_cast<int64_t>(B) * T * cfg->num_heads * cfg->head_v > 0x7fffffffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "B * T * num_heads * dv is too large");
    KDA_TRY(need_vec(q, "q"));
    KDA_TRY(need_vec(k, "k"));
    KDA_TRY(need_vec(v, "v"));
    KDA_TRY(need_vec(z, "z"));
    KDA_TRY(need_vec(g, "g"));
    KDA_TRY(need_idx(beta, 4, "beta"));
    KDA_TRY(need_vec(conv_w, "conv_w"));
    KDA_TRY(need_vec(norm_w, "norm_w"));
    KDA_TRY(need_vec(state_pool, "state_pool"));
    KDA_TRY(need_vec(conv_pool, "conv_pool"));
    KDA_TRY(need_idx(slot, 4, "slot"));
    KDA_TRY(need_vec(out, "out"));
    if (token_state) KDA_TRY(need_vec(token_state, "token_state"));
    if (token_conv) KDA_TRY(need_vec(token_conv, "token_conv"));
    kda::DecodeParams p;
    p.B = B;
    p.H = cfg->num_heads;
    p.num_slots = num_slots;
    p.T = T;
    p.token_state = token_state;
    p.token_conv = token_conv;
    p.q = q;
    p.k = k;
    p.v = v;
    p.z = z;
    p.g = g;
    p.beta = beta;
    p.conv_w = conv_w;
    p.norm_w = norm_w;
    p.state = state_pool;
    p.conv = conv_pool;
    p.slot = slot;
    p.out = out;
    p.l2_eps = cfg->l2_eps;
    p.rms_eps = cfg->rms_eps;
    return hip_status(kda::launch_decode(cfg->head_k, cfg->head_v, cfg->act_dtype, cfg->state_dtype, p,
                                         static_cast<hipStream_t>(stream)),
                      "decode launch");
}

}  // namespace

kda_status kda_decode_step(const kda_config* cfg, int32_t B, const void* q, const void* k, const void* v,
                           const void* z, const float* g, const float* beta, const float* conv_w,
                           const float* norm_w, void* state_pool, void* conv_pool, int32_t num_slots,
                           const int32_t* slot, void* out, void* stream) {
    return decode_common(cfg, B, 1, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool, num_slots, slot,
                         out, nullptr, nullptr, stream);
}

kda_status kda_decode_multi(const kda_config* cfg, int32_t B, int32_t T, const void* q, const void* k,
                            const void* v, const void* z, const float* g, const float* beta, const float* conv_w,
                            const float* norm_w, void* state_pool, void* conv_pool, int32_t num_slots,
                            const int32_t* slot, void* out, void* token_state, void* token_conv, void* stream) {
    return decode_common(cfg, B, T, q, k, v, z, g, beta, conv_w, norm_w, state_pool, conv_pool, num_slots, slot,
                         out, token_state, token_conv, stream);
}

namespace {

kda_status check_prefill_mode(int32_t ckpt_interval, int32_t flags) {
    if (ckpt_interval < 0 || ckpt_interval % 64 != 0)
        return fail(KDA_ERR_INVALID_ARG, "ckpt_interval must be 0 or a positive multiple of 64 (got %d)",
                    ckpt_interval);
    if (flags & ~(KDA_PREFILL_SPLIT | KDA_PREFILL_PAIRED | KDA_PREFILL_PAIRED_POLL_ONCE | KDA_PREFILL_CONV_DONE))
        return fail(KDA_ERR_INVALID_ARG, "unknown prefill flags 0x%x", flags);
    if ((flags & KDA_PREFILL_PAIRED_POLL_ONCE) && !(flags & KDA_PREFILL_PAIRED))
        return fail(KDA_ERR_INVALID_ARG, "KDA_PREFILL_PAIRED_POLL_ONCE needs KDA_PREFILL_PAIRED");
    if ((flags & KDA_PREFILL_SPLIT) && ckpt_interval == 0)
        return fail(KDA_ERR_INVALID_ARG, "KDA_PREFILL_SPLIT needs ckpt_interval > 0");
    if ((flags & KDA_PREFILL_SPLIT) && (flags & KDA_PREFILL_PAIRED))
        return fail(KDA_ERR_INVALID_ARG, "KDA_PREFILL_SPLIT and KDA_PREFILL_PAIRED exclude each other");
    return KDA_OK;
}

kda::PrefillWorkspace workspace_layout(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                                       int32_t ckpt_interval, int32_t flags) {
    return kda::prefill_workspace(num_seqs, cfg->num_heads, total_tokens, cfg->head_k, cfg->head_v,
                                  cfg->act_dtype == KDA_BF16 ? 2 : 4, ckpt_interval,
                                  (flags & KDA_PREFILL_SPLIT) != 0, (flags & KDA_PREFILL_PAIRED) != 0);
}

}  // namespace

size_t kda_prefill_workspace_bytes(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                                   int32_t ckpt_interval, int32_t flags) {
    if (check_cfg(cfg) != KDA_OK) return 0;
    if (num_seqs < 0 || total_tokens < 0) {
        fail(KDA_ERR_INVALID_ARG, "num_seqs and total_tokens must be >= 0");
        return 0;
    }
    if (check_prefill_mode(ckpt_interval, flags) != KDA_OK) return 0;
    const kda::PrefillWorkspace w = workspace_layout(cfg, num_seqs, total_tokens, ckpt_interval, flags);
    if (w.bytes == 0 && num_seqs > 0) fail(KDA_ERR_INVALID_ARG, "too many sequences or segments");
    return w.bytes;
}

kda_status kda_prefill_varlen(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens,
                              const int32_t* cu_seqlens, const int64_t* start_pos, const void* q,
                              const void* k, const void* v, const void* z, const float* g, const float* beta,
                              const float* conv_w, const float* norm_w, void* state_pool, void* conv_pool,
                              int32_t num_slots, const int32_t* init_slot, const int32_t* final_slot,
                              int32_t ckpt_interval, void* ckpt_state, void* ckpt_conv,
                              int32_t num_ckpt_slots, const int32_t* ckpt_base, int32_t flags, void* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    KDA_TRY(check_cfg(cfg));
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
    if (total_tokens < 0 || total_tokens > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "total_tokens must be in [0, 2^31) (got %lld)",
                    static_cast<long long>(total_tokens));
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1 (got %d)", num_slots);
    KDA_TRY(check_prefill_mode(ckpt_interval, flags));
    if (!kda::prefill_supported(cfg->head_k, cfg->head_v, cfg->act_dtype))
        return fail(KDA_ERR_UNSUPPORTED, "prefill does not support dk=%d dv=%d act_dtype=%d", cfg->head_k,
                    cfg->head_v, cfg->act_dtype);
    if ((flags & KDA_PREFILL_CONV_DONE) && cfg->act_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "KDA_PREFILL_CONV_DONE needs bf16 activations (act_dtype = KDA_BF16)");
    if (num_seqs == 0) return ok();
    KDA_TRY(need_idx(cu_seqlens, 4, "cu_seqlens"));
    if (start_pos) KDA_TRY(need_idx(start_pos, 8, "start_pos"));
    if (init_slot) KDA_TRY(need_idx(init_slot, 4, "init_slot"));
    if (final_slot) KDA_TRY(need_idx(final_slot, 4, "final_slot"));
    if (total_tokens > 0) {
        KDA_TRY(need_vec(q, "q"));
        KDA_TRY(need_vec(k, "k"));
        KDA_TRY(need_vec(v, "v"));
        KDA_TRY(need_vec(z, "z"));
        KDA_TRY(need_vec(g, "g"));
        KDA_TRY(need_idx(beta, 4, "beta"));
        KDA_TRY(need_vec(out, "out"));
    }
    KDA_TRY(need_vec(conv_w, "conv_w"));
    KDA_TRY(need_vec(norm_w, "norm_w"));
    KDA_TRY(need_vec(state_pool, "state_pool"));
    KDA_TRY(need_vec(conv_pool, "conv_pool"));
    if (ckpt_interval > 0) {
        if (num_ckpt_slots < 1)
            return fail(KDA_ERR_INVALID_ARG, "num_ckpt_slots must be >= 1 when checkpoints are on");
        KDA_TRY(need_vec(ckpt_state, "ckpt_state"));
        KDA_TRY(need_vec(ckpt_conv, "ckpt_conv"));
        KDA_TRY(need_idx(ckpt_base, 4, "ckpt_base"));
    }
    const kda::PrefillWorkspace wl = workspace_layout(cfg, num_seqs, total_tokens, ckpt_interval, flags);
    const size_t need = wl.bytes;
    if (need == 0) return fail(KDA_ERR_INVALID_ARG, "too many sequences or segments");
    const bool split = (flags & KDA_PREFILL_SPLIT) != 0;
    if (split && static_cast<int64_t>(wl.max_items) * 2 * cfg->num_heads > 0xffffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "too many segments x heads for one launch");
    if (workspace_bytes < need)
        return fail(KDA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    if (need > 0) KDA_TRY(need_vec(workspace, "workspace"));

    kda::PrefillParams p;
    p.N = num_seqs;
    p.H = cfg->num_heads;
    p.T = total_tokens;
    p.cu_seqlens = cu_seqlens;
    p.start_pos = start_pos;
    p.q = q;
    p.k = k;
    p.v = v;
    p.z = z;
    p.g = g;
    p.beta = beta;
    p.conv_w = conv_w;
    p.norm_w = norm_w;
    p.state = state_pool;
    p.conv = conv_pool;
    p.num_slots = num_slots;
    p.init_slot = init_slot;
    p.final_slot = final_slot;
    p.ckpt_interval = ckpt_interval;
    p.ckpt_state = ckpt_interval > 0 ? ckpt_state : nullptr;
    p.ckpt_conv = ckpt_interval > 0 ? ckpt_conv : nullptr;
    p.num_ckpt_slots = ckpt_interval > 0 ? num_ckpt_slots : 0;
    p.ckpt_base = ckpt_interval > 0 ? ckpt_base : nullptr;
    p.out = out;
    char* ws = static_cast<char*>(workspace);
    p.work = reinterpret_cast<kda::SeqWork*>(ws + wl.items);
    p.l2_eps = cfg->l2_eps;
    p.rms_eps = cfg->rms_eps;
    p.split = split ? 1 : 0;
    p.max_items = wl.max_items;
    p.seq_items = split ? reinterpret_cast<int2*>(ws + wl.seq_items) : nullptr;
    p.seg_F = split ? reinterpret_cast<float*>(ws + wl.seg_F) : nullptr;
    p.seg_G = split ? reinterpret_cast<float*>(ws + wl.seg_G) : nullptr;
    p.seg_S = split ? reinterpret_cast<float*>(ws + wl.seg_S) : nullptr;
    p.seq_x0 = split ? static_cast<void*>(ws + wl.seq_x0) : nullptr;
    p.state_bf16 = cfg->state_dtype == KDA_BF16 ? 1 : 0;
    p.ring = nullptr;
    p.ring_ctr = nullptr;
    p.max_pairs = 0;
    p.sched_grid = 0;
    p.spin_limit = (flags & KDA_PREFILL_PAIRED_POLL_ONCE) ? 1 : kda::PAIR_SPIN_LIMIT;
    p.conv_done = (flags & KDA_PREFILL_CONV_DONE) ? 1 : 0;
    p.status = reinterpret_cast<int32_t*>(ws + wl.status);
    if (wl.ring > 0) {
        // a scheduled launch needs a grid of at least 16 workgroups that the
        // device holds at once; otherwise the one-workgroup kernel runs
        const int64_t chains = static_cast<int64_t>(num_seqs) * cfg->num_heads;
        const int64_t grid = kda::pair_grid(chains, kda::prefill_pair_capacity(cfg->head_k, cfg->act_dtype));
        if (grid >= 16) {
            p.ring = ws + wl.ring;
            p.ring_ctr = reinterpret_cast<int32_t*>(ws + wl.ring_ctr);
            p.max_pairs = wl.max_pairs;
            p.sched_grid = static_cast<int32_t>(grid);
        }
    }
    return hip_status(kda::launch_prefill(cfg->head_k, cfg->head_v, cfg->act_dtype, p,
                                          static_cast<hipStream_t>(stream)),
                      "prefill launch");
}

kda_status kda_project_inputs(const kda_config* cfg, int32_t T, int32_t Dm, const void* x, const void* w, void* q,
                              void* k, void* v, void* z, float* g, float* beta, void* stream) {
    KDA_TRY(check_cfg(cfg));
    if (cfg->act_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "input projections need bf16 activations (act_dtype = KDA_BF16)");
    if (T < 0) return fail(KDA_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (Dm < 64 || Dm % 64 != 0) return fail(KDA_ERR_INVALID_ARG, "Dm must be a positive multiple of 64 (got %d)", Dm);
    if (Dm > (1 << 22)) return fail(KDA_ERR_INVALID_ARG, "Dm must be at most 4194304 (got %d)", Dm);
    const int64_t N = static_cast<int64_t>(cfg->num_heads) * (3 * cfg->head_k + 2 * cfg->head_v) + cfg->num_heads;
    if (N * Dm * 2 >= (1LL << 31) * 2 || static_cast<int64_t>(T) * Dm * 2 >= (1LL << 40))
        return fail(KDA_ERR_INVALID_ARG, "projection sizes too large");
    if (T == 0) return ok();
    KDA_TRY(need_vec(x, "x"));
    KDA_TRY(need_vec(w, "w"));
    KDA_TRY(need_vec(q, "q"));
    KDA_TRY(need_vec(k, "k"));
    KDA_TRY(need_vec(v, "v"));
    KDA_TRY(need_vec(z, "z"));
    KDA_TRY(need_vec(g, "g"));
    KDA_TRY(need_idx(beta, 4, "beta"));
    kda::ProjectParams p{};
    p.T = T;
    p.N = static_cast<int32_t>(N);
    p.Dm = Dm;
    p.mode = 0;
    p.H = cfg->num_heads;
    p.dk = cfg->head_k;
    p.dv = cfg->head_v;
    p.x = x;
    p.w = w;
    p.q = q;
    p.k = k;
    p.v = v;
    p.z = z;
    p.g = g;
    p.beta = beta;
    return hip_status(kda::launch_project(p, static_cast<hipStream_t>(stream)), "projection launch");
}

kda_status kda_project_inputs_conv(const kda_config* cfg, int32_t num_seqs, int32_t T, int32_t Dm,
                                   const int32_t* cu_seqlens, const void* x, const void* w, const float* conv_w,
                                   const void* conv_pool, int32_t num_slots, const int32_t* init_slot, void* q,
                                   void* k, void* v, void* z, float* g, float* beta, void* stream) {
    KDA_TRY(check_cfg(cfg));
    if (cfg->act_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "input projections need bf16 activations (act_dtype = KDA_BF16)");
    if (num_seqs < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", num_seqs);
    if (T < 0) return fail(KDA_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1 (got %d)", num_slots);
    if (Dm < 64 || Dm % 64 != 0) return fail(KDA_ERR_INVALID_ARG, "Dm must be a positive multiple of 64 (got %d)", Dm);
    if (Dm > (1 << 22)) return fail(KDA_ERR_INVALID_ARG, "Dm must be at most 4194304 (got %d)", Dm);
    const int64_t N = static_cast<int64_t>(cfg->num_heads) * (3 * cfg->head_k + 2 * cfg->head_v) + cfg->num_heads;
    if (N * Dm * 2 >= (1LL << 31) * 2 || static_cast<int64_t>(T) * Dm * 2 >= (1LL << 40))
        return fail(KDA_ERR_INVALID_ARG, "projection sizes too large");
    if (T == 0) return ok();
    KDA_TRY(need_idx(cu_seqlens, 4, "cu_seqlens"));
    KDA_TRY(need_vec(x, "x"));
    KDA_TRY(need_vec(w, "w"));
    KDA_TRY(need_vec(conv_w, "conv_w"));
    KDA_TRY(need_vec(conv_pool, "conv_pool"));
    if (init_slot) KDA_TRY(need_idx(init_slot, 4, "init_slot"));
    KDA_TRY(need_vec(q, "q"));
    KDA_TRY(need_vec(k, "k"));
    KDA_TRY(need_vec(v, "v"));
    KDA_TRY(need_vec(z, "z"));
    KDA_TRY(need_vec(g, "g"));
    KDA_TRY(need_idx(beta, 4, "beta"));
    kda::ProjectParams p{};
    p.T = T;
    p.N = static_cast<int32_t>(N);
    p.Dm = Dm;
    p.mode = 0;
    p.H = cfg->num_heads;
    p.dk = cfg->head_k;
    p.dv = cfg->head_v;
    p.x = x;
    p.w = w;
    p.q = q;
    p.k = k;
    p.v = v;
    p.z = z;
    p.g = g;
    p.beta = beta;
    p.conv = 1;
    p.num_seqs = num_seqs;
    p.cu_seqlens = cu_seqlens;
    p.init_slot = init_slot;
    p.conv_pool = conv_pool;
    p.num_slots = num_slots;
    p.conv_w = conv_w;
    return hip_status(kda::launch_project(p, static_cast<hipStream_t>(stream)), "projection launch");
}

kda_status kda_project_output(const kda_config* cfg, int32_t T, int32_t Dm, const void* o, const void* w_o, void* y,
                              void* stream) {
    KDA_TRY(check_cfg(cfg));
    if (cfg->act_dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "the output projection needs bf16 activations (act_dtype = KDA_BF16)");
    if (T < 0) return fail(KDA_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (Dm < 1) return fail(KDA_ERR_INVALID_ARG, "Dm must be >= 1 (got %d)", Dm);
    const int64_t K = static_cast<int64_t>(cfg->num_heads) * cfg->head_v;
    if (K % 64 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "the output projection needs num_heads * head_v to be a multiple of 64 (got %lld)",
                    static_cast<long long>(K));
    if (K > (1 << 22))
        return fail(KDA_ERR_INVALID_ARG, "num_heads * head_v must be at most 4194304 (got %lld)", static_cast<long long>(K));
    if (static_cast<int64_t>(Dm) * K * 2 >= (1LL << 32) || static_cast<int64_t>(T) * K * 2 >= (1LL << 40))
        return fail(KDA_ERR_INVALID_ARG, "projection sizes too large");
    if (T == 0) return ok();
    KDA_TRY(need_vec(o, "o"));
    KDA_TRY(need_vec(w_o, "w_o"));
    KDA_TRY(need_idx(y, 2, "y"));
    kda::ProjectParams p{};
    p.T = T;
    p.N = Dm;
    p.Dm = static_cast<int32_t>(K);
    p.H = cfg->num_heads;
    p.dk = cfg->head_k;
    p.dv = cfg->head_v;
    p.mode = 1;
    p.x = o;
    p.w = w_o;
    p.y = y;
    return hip_status(kda::launch_project(p, static_cast<hipStream_t>(stream)), "output projection launch");
}

kda_status kda_state_checkpoint(const kda_config* cfg, int32_t n, const void* state_pool, const void* conv_pool,
                                int32_t num_slots, const int32_t* src_slot, void* ckpt_state, void* ckpt_conv,
                                int32_t num_ckpt_slots, const int32_t* dst_ckpt, void* stream) {
    KDA_TRY(check_copy_args(cfg, n, state_pool, conv_pool, num_slots, src_slot, ckpt_state, ckpt_conv,
                            num_ckpt_slots, dst_ckpt));
    if (n == 0) return ok();
    const kda::CopyParams p = copy_params(cfg, n, state_pool, conv_pool, num_slots, src_slot, ckpt_state,
                                          ckpt_conv, num_ckpt_slots, dst_ckpt);
    return hip_status(kda::launch_copy(p, static_cast<hipStream_t>(stream)), "checkpoint copy launch");
}

kda_status kda_resume(const kda_config* cfg, int32_t n, const void* ckpt_state, const void* ckpt_conv,
                      int32_t num_ckpt_slots, const int32_t* src_ckpt, void* state_pool, void* conv_pool,
                      int32_t num_slots, const int32_t* dst_slot, void* stream) {
    KDA_TRY(check_copy_args(cfg, n, ckpt_state, ckpt_conv, num_ckpt_slots, src_ckpt, state_pool, conv_pool,
                            num_slots, dst_slot));
    if (n == 0) return ok();
    const kda::CopyParams p = copy_params(cfg, n, ckpt_state, ckpt_conv, num_ckpt_slots, src_ckpt, state_pool,
                                          conv_pool, num_slots, dst_slot);
    return hip_status(kda::launch_copy(p, static_cast<hipStream_t>(stream)), "resume copy launch");
}

}  // extern "C"
