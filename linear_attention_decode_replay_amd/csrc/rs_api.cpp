// Host side of the C ABI declared in replayssm.h: argument validation, the
// paged block layout, the per-row cursor/flush metadata and kernel launch.
// The entry points allocate no device memory.  Global state: the error text
// (thread-local) and, in rs_kernels.hip, a mutex-guarded cache of occupancy
// queries (workgroups per compute unit of the persistent replay step, per
// device and LDS size), which grows on the host heap the first time each
// (kernel, LDS size, device) is launched.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "replayssm.h"
#include "rs_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return RS_OK;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int dtype_bytes(int dt) { return dt == RS_F32 ? 4 : (dt == RS_E4M3 ? 1 : 2); }

const int kMaxL = 64;

bool two_precision(const rs_layer& L) { return L.read_dtype >= 0 && L.read_dtype != L.state_dtype; }

// Key groups: n_groups, or one per head.
int groups_of(const rs_layer& L) { return L.n_groups > 0 ? L.n_groups : L.n_heads; }
// Key record slots per group: the ring's, plus, on a speculative layer whose
// keys are shared by several heads, T more that hold the drafts of a flushing
// row until replay_spec_commit moves them to slot 0 (the other heads of the
// group may still be reading the committed keys there during the verify).
int key_slots_of(const rs_layer& L) {
    const int slots = L.spec_T > 0 ? L.L : L.L - 1;
    return L.spec_T > 0 && groups_of(L) != L.n_heads ? slots + L.spec_T : slots;
}
// LDS of one workgroup on gfx950, the one target the kernels are built for;
// a launch also checks the device's own limit (do_launch).
const size_t kMaxLds = 160 * 1024;
// LDS any gfx9 workgroup can have without asking the device.
const size_t kBaseLds = 64 * 1024;

int check_layer(const rs_layer* L, rs::Kind kind) {
    if (!L) return fail(RS_EINVAL, "layer is NULL");
    if (L->form != RS_MAMBA2 && L->form != RS_GDN) return fail(RS_EINVAL, "unknown form %d", L->form);
    if (L->n_heads < 1) return fail(RS_EINVAL, "n_heads must be >= 1 (got %d)", L->n_heads);
    if (L->d_v < 1 || L->d_k < 1) return fail(RS_EINVAL, "d_v and d_k must be >= 1");
    if (L->L < 1 || L->L > kMaxL) return fail(RS_EINVAL, "L must be in 1..%d (got %d)", kMaxL, L->L);
    for (int dt : {L->state_dtype, L->record_dtype, L->io_dtype})
        if (dt != RS_F32 && dt != RS_F16 && dt != RS_BF16) return fail(RS_EINVAL, "unknown dtype %d", dt);
    if (L->state_dtype == RS_BF16) return fail(RS_EUNSUPPORTED, "bf16 state is not supported");
    if (L->read_dtype < -1 || L->read_dtype > RS_E4M3) return fail(RS_EINVAL, "unknown read dtype %d", L->read_dtype);
    if (two_precision(*L)) {
        if (L->form != RS_MAMBA2)
            return fail(RS_EUNSUPPORTED, "two-precision checkpoint: Mamba-2 form only (a GDN read copy would "
                                         "leak into the buffered corrected values)");
        if (L->state_dtype != RS_F32 && !(L->state_dtype == RS_F16 && L->read_dtype == RS_E4M3))
            return fail(RS_EUNSUPPORTED, "two-precision checkpoint: an fp32 recurrence copy, or an fp16 one with "
                                         "an E4M3 read copy");
    }
    if (L->record_dtype == RS_BF16) return fail(RS_EUNSUPPORTED, "bf16 records are not supported");
    if (L->state_rounding != RS_ROUND_NEAREST && L->state_rounding != RS_ROUND_STOCHASTIC)
        return fail(RS_EINVAL, "unknown state rounding %d", L->state_rounding);
    if (L->state_rounding == RS_ROUND_STOCHASTIC && L->state_dtype != RS_F16)
        return fail(RS_EUNSUPPORTED, "stochastic rounding: an fp16 checkpoint / state (recurrence copy) only");
    if (L->gdn_route != RS_GDN_OUTPUT_ONLY && L->gdn_route != RS_GDN_RECONSTRUCT)
        return fail(RS_EINVAL, "unknown Gated DeltaNet route %d", L->gdn_route);
    if (L->gdn_route == RS_GDN_RECONSTRUCT && L->form != RS_GDN)
        return fail(RS_EINVAL, "the state-reconstruction route is a Gated DeltaNet option");
    if (L->n_groups < 0 || (L->n_groups > 0 && L->n_heads % L->n_groups != 0))
        return fail(RS_EINVAL, "n_groups (%d) must be 0 or divide n_heads (%d)", L->n_groups, L->n_heads);
    const bool spec_kind = kind == rs::Kind::SpecVerify || kind == rs::Kind::SpecCommit;
    if (L->spec_T != 0) {
        const int T = L->spec_T;
        if (T < 1 || T > L->L) return fail(RS_EINVAL, "spec_T must be in 1..L (got %d, L=%d)", T, L->L);
        if (T != 1 && T != 2 && T != 4 && T != 8)
            return fail(RS_EUNSUPPORTED, "spec_T must be 1, 2, 4 or 8 (got %d)", T);
        if (two_precision(*L) && (L->form != RS_MAMBA2 || L->state_dtype != RS_F32))
            return fail(RS_EUNSUPPORTED, "speculative verify with a read copy: Mamba-2 with an fp32 recurrence "
                                         "copy only");
        if (kind == rs::Kind::ReplayStep)
            return fail(RS_EINVAL, "a speculative layer (spec_T=%d) is stepped with replay_spec_verify", T);
    } else if (spec_kind) {
        return fail(RS_EINVAL, "replay_spec_verify / replay_spec_commit need a speculative layer (spec_T > 0)");
    }
    if (!rs::compiled(kind, *L)) {
        if (spec_kind)
            return fail(RS_EUNSUPPORTED, "no speculative kernel for d_v=%d d_k=%d (supported: 16x32, 64x128, 128x128)",
                        L->d_v, L->d_k);
        if (L->read_dtype == RS_E4M3)
            return fail(RS_EUNSUPPORTED, "no kernel for an E4M3 read copy with d_v=%d d_k=%d (supported: 64x128, "
                                         "128x128)", L->d_v, L->d_k);
        return fail(RS_EUNSUPPORTED, "no kernel for d_v=%d d_k=%d (supported: 16x32, 64x128, 128x128)",
                    L->d_v, L->d_k);
    }
    if (rs::lds_bytes(kind, *L) > kMaxLds)
        return fail(RS_EUNSUPPORTED, "buffer of L=%d records needs %zu bytes of LDS (> %zu)", L->L,
                    rs::lds_bytes(kind, *L), kMaxLds);
    return RS_OK;
}

void layout_of(const rs_layer& L, rs_block_layout* o) {
    // a speculative ring holds up to L committed records; a standard buffer
    // L - 1 (the L-th token of a window flushes without being stored)
    const int64_t slots = L.spec_T > 0 ? L.L : L.L - 1;
    const int64_t H = L.n_heads;
    const int64_t sb = dtype_bytes(L.state_dtype), rb = dtype_bytes(L.record_dtype);
    o->ckpt_off = 0;
    o->rec_x_off = align_up(H * L.d_v * L.d_k * sb, 256);
    o->rec_k_off = align_up(o->rec_x_off + H * slots * L.d_v * rb, 256);
    o->rec_lam_off = align_up(o->rec_k_off + (int64_t)groups_of(L) * key_slots_of(L) * L.d_k * rb, 256);
    o->block_bytes = align_up(o->rec_lam_off + H * slots * 4, 256);
    o->ckpt_lo_off = 0;
    o->ckpt_scale_off = 0;
    if (two_precision(L)) {
        o->ckpt_lo_off = o->block_bytes;
        o->block_bytes = align_up(o->ckpt_lo_off + H * L.d_v * L.d_k * dtype_bytes(L.read_dtype), 256);
        if (L.read_dtype == RS_E4M3) {
            o->ckpt_scale_off = o->block_bytes;
            o->block_bytes = align_up(o->ckpt_scale_off + H * L.d_v * 4, 256);
        }
    }
    o->slots = (int32_t)slots;
    o->key_slots = key_slots_of(L);
}

int check_batch(const rs_layer& L, const rs_batch* b, bool needs_cursor, bool needs_flush) {
    if (!b) return fail(RS_EINVAL, "batch is NULL");
    if (b->n_rows < 0) return fail(RS_EINVAL, "n_rows must be >= 0");
    if (b->n_rows == 0) return RS_OK;
    if (b->n_rows > 65535) return fail(RS_EINVAL, "n_rows must be <= 65535 (got %d)", b->n_rows);
    if (b->n_blocks < 1) return fail(RS_EINVAL, "n_blocks must be >= 1");
    if (!b->pool || !aligned(b->pool, 256)) return fail(RS_EINVAL, "pool must be non-NULL and 256-byte aligned");
    if (!b->block_table || !aligned(b->block_table, 4))
        return fail(RS_EINVAL, "block_table must be non-NULL and 4-byte aligned");
    if (needs_cursor && !b->write_pos) return fail(RS_EINVAL, "write_pos is NULL");
    if (b->write_pos && !aligned(b->write_pos, 4)) return fail(RS_EINVAL, "write_pos must be 4-byte aligned");
    if (needs_flush && !b->flush) return fail(RS_EINVAL, "flush is NULL");
    if (b->flush && !aligned(b->flush, 4)) return fail(RS_EINVAL, "flush must be 4-byte aligned");
    if (b->err_count && !aligned(b->err_count, 4)) return fail(RS_EINVAL, "err_count is misaligned");
    if (b->next_write_pos && !aligned(b->next_write_pos, 4))
        return fail(RS_EINVAL, "next_write_pos must be 4-byte aligned");
    if (b->next_write_pos && b->next_write_pos == b->write_pos)
        return fail(RS_EINVAL, "next_write_pos must not alias write_pos");
    if (b->flush_hint < RS_FLUSH_UNKNOWN || b->flush_hint > RS_FLUSH_MIXED)
        return fail(RS_EINVAL, "unknown flush_hint %d", b->flush_hint);
    return RS_OK;
}

int check_vec(const char* name, const void* p, int64_t rs, int64_t hs, int d, int elem) {
    if (!p) return fail(RS_EINVAL, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(RS_EINVAL, "%s must be 16-byte aligned", name);
    if ((rs * elem) % 16 || (hs * elem) % 16)
        return fail(RS_EINVAL, "%s strides (%lld, %lld elements) must keep 16-byte alignment", name,
                    (long long)rs, (long long)hs);
    if (hs < d || rs < 0) return fail(RS_EINVAL, "%s strides (%lld, %lld) overlap a %d-vector", name,
                                      (long long)rs, (long long)hs, d);
    return RS_OK;
}

int check_io(const rs_layer& L, const rs_batch& b, const rs_step_io* io) {
    if (!io) return fail(RS_EINVAL, "io is NULL");
    if (b.n_rows == 0) return RS_OK;
    const int e = dtype_bytes(L.io_dtype);
    int rc;
    const int64_t G = groups_of(L);
    if ((rc = check_vec("q", io->q, io->q_row_stride, io->q_head_stride, L.d_k, e))) return rc;
    if ((rc = check_vec("k", io->k, io->k_row_stride, io->k_head_stride, L.d_k, e))) return rc;
    if ((rc = check_vec("v", io->v, io->v_row_stride, io->v_head_stride, L.d_v, e))) return rc;
    if (b.n_rows > 1) {
        if (io->q_row_stride < G * io->q_head_stride || io->k_row_stride < G * io->k_head_stride ||
            io->v_row_stride < (int64_t)L.n_heads * io->v_head_stride)
            return fail(RS_EINVAL, "row strides overlap the heads of the previous row");
    }
    if (!io->log_decay || !aligned(io->log_decay, 16)) return fail(RS_EINVAL, "log_decay must be non-NULL and 16-byte aligned");
    if (L.form == RS_GDN && (!io->beta || !aligned(io->beta, 16)))
        return fail(RS_EINVAL, "beta must be non-NULL and 16-byte aligned for Gated DeltaNet");
    if (!io->out || !aligned(io->out, 16)) return fail(RS_EINVAL, "out must be non-NULL and 16-byte aligned");
    return RS_OK;
}

rs::StepParams params(const rs_layer& L, const rs_batch& b) {
    rs_block_layout lay;
    layout_of(L, &lay);
    rs::StepParams p{};
    p.pool = static_cast<char*>(b.pool);
    p.block_bytes = lay.block_bytes;
    p.n_blocks = b.n_blocks;
    p.ckpt_off = lay.ckpt_off;
    p.recx_off = lay.rec_x_off;
    p.reck_off = lay.rec_k_off;
    p.reclam_off = lay.rec_lam_off;
    p.ckpt_lo_off = lay.ckpt_lo_off;
    p.ckpt_sc_off = lay.ckpt_scale_off;
    p.block_table = b.block_table;
    p.write_pos = b.write_pos;
    p.flush = b.flush;
    p.err = b.err_count;
    p.next_wp = nullptr;
    p.n_rows = b.n_rows;
    p.n_heads = L.n_heads;
    p.L = L.L;
    p.slots = lay.slots;
    p.key_slots = lay.key_slots;
    p.key_bytes = L.d_k * dtype_bytes(L.record_dtype);
    p.heads_per_group = L.n_heads / groups_of(L);
    p.sr = L.state_rounding == RS_ROUND_STOCHASTIC;
    p.reconstruct = L.gdn_route == RS_GDN_RECONSTRUCT;
    // (the state-reconstruction route has one kernel for every row)
    p.flush_hint = p.reconstruct ? RS_FLUSH_UNKNOWN : b.flush_hint;
    p.sr_key0 = b.sr_key0;
    p.sr_key1 = b.sr_key1;
    p.sr_step = b.sr_step;
    return p;
}

void set_io(rs::StepParams& p, const rs_step_io& io) {
    p.q = io.q;
    p.k = io.k;
    p.v = io.v;
    p.qs_r = io.q_row_stride;
    p.qs_h = io.q_head_stride;
    p.ks_r = io.k_row_stride;
    p.ks_h = io.k_head_stride;
    p.vs_r = io.v_row_stride;
    p.vs_h = io.v_head_stride;
    p.lam = io.log_decay;
    p.beta = io.beta;
    p.out = io.out;
}

int do_launch(rs::Kind kind, const rs_layer& L, const rs::StepParams& p, hipStream_t stream) {
    const size_t lds = rs::lds_bytes(kind, L);
    if (lds > kBaseLds) {
        int dev = 0, max_lds = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return fail(RS_EHIP, "cannot query the device's LDS per workgroup");
        if (lds > (size_t)max_lds)
            return fail(RS_EUNSUPPORTED, "buffer of L=%d records needs %zu bytes of LDS; device %d allows %d",
                        L.L, lds, dev, max_lds);
    }
    (void)hipGetLastError();  // do not report an earlier, unrelated error as ours
    const hipError_t e = rs::launch(kind, L, p, stream);
    if (e != hipSuccess) return fail(RS_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// The step kind that defines a layer: standard decoding, or the verify step
// of a speculative layer.
rs::Kind step_kind(const rs_layer* layer) {
    return layer && layer->spec_T != 0 ? rs::Kind::SpecVerify : rs::Kind::ReplayStep;
}

}  // namespace

extern "C" {

int rs_block_layout_get(const rs_layer* layer, rs_block_layout* out) {
    int rc = check_layer(layer, step_kind(layer));
    if (rc) return rc;
    if (!out) return fail(RS_EINVAL, "out is NULL");
    layout_of(*layer, out);
    return ok();
}

int rs_layer_supported(const rs_layer* layer) {
    int rc = check_layer(layer, step_kind(layer));
    if (rc) return rc;
    rc = check_layer(layer, rs::Kind::ConventionalStep);
    return rc ? rc : ok();
}

int replay_decode_step(const rs_layer* layer, const rs_batch* batch, const rs_step_io* io,
                       hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::ReplayStep))) return rc;
    if ((rc = check_batch(*layer, batch, true, false))) return rc;
    if ((rc = check_io(*layer, *batch, io))) return rc;
    if (batch->n_rows == 0) return ok();
    rs::StepParams p = params(*layer, *batch);
    p.next_wp = batch->next_write_pos;
    set_io(p, *io);
    return do_launch(rs::Kind::ReplayStep, *layer, p, stream);
}

int replay_flush(const rs_layer* layer, const rs_batch* batch, hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::Flush))) return rc;
    if ((rc = check_batch(*layer, batch, true, true))) return rc;
    if (batch->n_rows == 0) return ok();
    const rs::StepParams p = params(*layer, *batch);
    return do_launch(rs::Kind::Flush, *layer, p, stream);
}

int conventional_decode_step(const rs_layer* layer, const rs_batch* batch, const rs_step_io* io,
                             hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::ConventionalStep))) return rc;
    if ((rc = check_batch(*layer, batch, false, false))) return rc;
    if ((rc = check_io(*layer, *batch, io))) return rc;
    if (batch->n_rows == 0) return ok();
    rs::StepParams p = params(*layer, *batch);
    p.write_pos = nullptr;
    p.flush = nullptr;
    set_io(p, *io);
    return do_launch(rs::Kind::ConventionalStep, *layer, p, stream);
}

int replay_state_reset(const rs_layer* layer, const rs_batch* batch, const uint8_t* mask,
                       hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::Reset))) return rc;
    if ((rc = check_batch(*layer, batch, false, false))) return rc;
    if (batch->n_rows == 0) return ok();
    if (!mask || !aligned(mask, 4)) return fail(RS_EINVAL, "mask must be non-NULL and 4-byte aligned");
    rs::StepParams p = params(*layer, *batch);
    p.mask = mask;
    return do_launch(rs::Kind::Reset, *layer, p, stream);
}

int rs_meta_step(int32_t L, int32_t n_rows, const int32_t* steps_since_anchor,
                 const uint8_t* force_flush, int32_t* write_pos, uint8_t* flush) {
    if (L < 1 || L > kMaxL) return fail(RS_EINVAL, "L must be in 1..%d (got %d)", kMaxL, L);
    if (n_rows < 0) return fail(RS_EINVAL, "n_rows must be >= 0");
    if (n_rows == 0) return ok();
    if (!steps_since_anchor || !write_pos || !flush) return fail(RS_EINVAL, "NULL array");
    for (int32_t r = 0; r < n_rows; ++r) {
        const int32_t n = steps_since_anchor[r];
        if (n < 0) {
            write_pos[r] = 0;
            flush[r] = 0;
            continue;
        }
        const int32_t w = n % L;
        write_pos[r] = w;
        flush[r] = (uint8_t)((w == L - 1) || (force_flush && force_flush[r]));
    }
    return ok();
}

int rs_meta_advance(int32_t L, int32_t n_rows, int32_t* steps_since_anchor, const uint8_t* flush) {
    if (L < 1 || L > kMaxL) return fail(RS_EINVAL, "L must be in 1..%d (got %d)", kMaxL, L);
    if (n_rows < 0) return fail(RS_EINVAL, "n_rows must be >= 0");
    if (n_rows == 0) return ok();
    if (!steps_since_anchor || !flush) return fail(RS_EINVAL, "NULL array");
    for (int32_t r = 0; r < n_rows; ++r) {
        if (steps_since_anchor[r] < 0) continue;
        steps_since_anchor[r] = flush[r] ? 0 : steps_since_anchor[r] + 1;
    }
    return ok();
}

int replay_spec_verify(const rs_layer* layer, const rs_batch* batch, const rs_spec_io* io, hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::SpecVerify))) return rc;
    if ((rc = check_batch(*layer, batch, true, false))) return rc;
    if (!io) return fail(RS_EINVAL, "io is NULL");
    if (batch->n_rows == 0) return ok();
    const int T = layer->spec_T, e = dtype_bytes(layer->io_dtype);
    const int64_t G = groups_of(*layer);  // q and k: one per key group
    struct { const char* name; const void* p; int64_t rs, ts, hs; int d; int64_t heads; } v3[] = {
        {"q", io->q, io->q_row_stride, io->q_token_stride, io->q_head_stride, layer->d_k, G},
        {"k", io->k, io->k_row_stride, io->k_token_stride, io->k_head_stride, layer->d_k, G},
        {"v", io->v, io->v_row_stride, io->v_token_stride, io->v_head_stride, layer->d_v, layer->n_heads}};
    for (const auto& a : v3) {
        if ((rc = check_vec(a.name, a.p, a.rs, a.hs, a.d, e))) return rc;
        if ((a.ts * e) % 16) return fail(RS_EINVAL, "%s token stride must keep 16-byte alignment", a.name);
        if (a.ts < a.heads * a.hs)
            return fail(RS_EINVAL, "%s token stride overlaps the heads of the previous token", a.name);
        if (batch->n_rows > 1 && a.rs < (int64_t)T * a.ts)
            return fail(RS_EINVAL, "%s row stride overlaps the tokens of the previous row", a.name);
    }
    if (!io->log_decay || !aligned(io->log_decay, 16))
        return fail(RS_EINVAL, "log_decay must be non-NULL and 16-byte aligned");
    if (!io->out || !aligned(io->out, 16)) return fail(RS_EINVAL, "out must be non-NULL and 16-byte aligned");
    if (layer->form == RS_GDN && (!io->beta || !aligned(io->beta, 16)))
        return fail(RS_EINVAL, "beta must be non-NULL and 16-byte aligned for Gated DeltaNet");
    rs::StepParams p = params(*layer, *batch);
    p.spec_T = T;
    p.beta = io->beta;
    p.q = io->q;
    p.k = io->k;
    p.v = io->v;
    p.qs_r = io->q_row_stride;
    p.qs_t = io->q_token_stride;
    p.qs_h = io->q_head_stride;
    p.ks_r = io->k_row_stride;
    p.ks_t = io->k_token_stride;
    p.ks_h = io->k_head_stride;
    p.vs_r = io->v_row_stride;
    p.vs_t = io->v_token_stride;
    p.vs_h = io->v_head_stride;
    p.lam = io->log_decay;
    p.out = io->out;
    return do_launch(rs::Kind::SpecVerify, *layer, p, stream);
}

int replay_spec_commit(const rs_layer* layer, const rs_batch* batch, const int32_t* accepted, uint8_t* next_flush,
                       hipStream_t stream) {
    int rc;
    if ((rc = check_layer(layer, rs::Kind::SpecCommit))) return rc;
    if ((rc = check_batch(*layer, batch, true, false))) return rc;
    if (batch->n_rows == 0) return ok();
    if (!accepted || !aligned(accepted, 4)) return fail(RS_EINVAL, "accepted must be non-NULL and 4-byte aligned");
    if (!batch->next_write_pos) return fail(RS_EINVAL, "next_write_pos is NULL");
    if (!next_flush) return fail(RS_EINVAL, "next_flush is NULL");
    if (batch->flush && (const void*)batch->flush == (const void*)next_flush)
        return fail(RS_EINVAL, "next_flush must not alias flush");
    rs::StepParams p = params(*layer, *batch);
    p.spec_T = layer->spec_T;
    p.next_wp = batch->next_write_pos;
    p.accepted = accepted;
    p.next_flush = next_flush;
    return do_launch(rs::Kind::SpecCommit, *layer, p, stream);
}

int rs_spec_meta_step(int32_t L, int32_t T, int32_t n_rows, const int32_t* committed, const uint8_t* force,
                      uint8_t* flush) {
    if (L < 1 || L > kMaxL) return fail(RS_EINVAL, "L must be in 1..%d (got %d)", kMaxL, L);
    if (T < 1 || T > L) return fail(RS_EINVAL, "T must be in 1..L (got %d)", T);
    if (n_rows < 0) return fail(RS_EINVAL, "n_rows must be >= 0");
    if (n_rows == 0) return ok();
    if (!committed || !flush) return fail(RS_EINVAL, "NULL array");
    for (int32_t r = 0; r < n_rows; ++r)
        flush[r] = (uint8_t)(committed[r] >= 0 && (committed[r] + T > L || (force && force[r])));
    return ok();
}

int rs_spec_meta_advance(int32_t L, int32_t T, int32_t n_rows, int32_t* committed, const uint8_t* flush,
                         const int32_t* accepted) {
    if (L < 1 || L > kMaxL) return fail(RS_EINVAL, "L must be in 1..%d (got %d)", kMaxL, L);
    if (T < 1 || T > L) return fail(RS_EINVAL, "T must be in 1..L (got %d)", T);
    if (n_rows < 0) return fail(RS_EINVAL, "n_rows must be >= 0");
    if (n_rows == 0) return ok();
    if (!committed || !flush || !accepted) return fail(RS_EINVAL, "NULL array");
    // every count is checked before any row moves, so a bad count leaves the
    // mirror as it was (the device commit skips and counts such a row)
    for (int32_t r = 0; r < n_rows; ++r)
        if (committed[r] >= 0 && (accepted[r] < 0 || accepted[r] > T))
            return fail(RS_EINVAL, "accepted[%d] = %d is outside 0..T (T=%d)", r, accepted[r], T);
    for (int32_t r = 0; r < n_rows; ++r)
        if (committed[r] >= 0) committed[r] = (flush[r] ? 0 : committed[r]) + accepted[r];
    return ok();
}

const char* rs_last_error(void) { return g_err; }

}  // extern "C"
