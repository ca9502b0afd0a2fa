// Internal interface between the host entry points (rs_api.cpp) and the
// kernels (rs_kernels.hip).  Not installed; the public ABI is replayssm.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "replayssm.h"

namespace rs {

// Everything a launch needs, passed to the kernels by value.
struct StepParams {
    char* pool;
    int64_t block_bytes;
    int64_t n_blocks;
    int64_t ckpt_off, recx_off, reck_off, reclam_off;
    int64_t ckpt_lo_off;    // read copy of a two-precision checkpoint (else unused)
    int64_t ckpt_sc_off;    // per-row scales of an E4M3 read copy (else unused)
    const int32_t* block_table;
    const int32_t* write_pos;
    const uint8_t* flush;   // per-row flag (replay step, token-less flush)
    const uint8_t* mask;    // per-row mask (state reset)
    int32_t* err;
    int32_t* next_wp;       // replay step: next cursor per row (optional)
    const void* q;
    const void* k;
    const void* v;
    int64_t qs_r, qs_h, ks_r, ks_h, vs_r, vs_h;
    const float* lam;
    const float* beta;
    float* out;
    int32_t n_rows, n_heads, L, slots;
    int32_t heads_per_group;   // heads sharing one key / query (1: per-head keys)
    int32_t sr;                // stochastic rounding of 16-bit state stores
    int32_t reconstruct;       // Gated DeltaNet: rebuild S_{t-1} on every step
    int32_t flush_hint;        // rs_flush_hint of the launch (see k_replay_step)
    int32_t meta_off;          // persistent replay step: LDS byte offsets of the rows' metadata
    int32_t defer_off;         //   and of the deferred writes,
    int32_t defer_cap;         //   and the items these hold
    uint64_t sr_key0, sr_key1, sr_step;
    // speculative verify / commit
    int32_t spec_T;
    int64_t qs_t, ks_t, vs_t;  // token strides (elements)
    const int32_t* accepted;   // commit: drafts accepted per row
    uint8_t* next_flush;       // commit: next step's flag per row
    int32_t key_slots;         // key record slots per group (slots, or L + T on a
                               // speculative layer with grouped keys)
    int32_t key_bytes;         // bytes of one key record (d_k * record size)
};

enum class Kind { ReplayStep, ConventionalStep, Flush, Reset, SpecVerify, SpecCommit };

// Dynamic LDS bytes a launch of `kind` needs for this layer (0 if none).
size_t lds_bytes(Kind kind, const rs_layer& layer);

// True if a kernel of `kind` is compiled for this layer.
bool compiled(Kind kind, const rs_layer& layer);

// Launch; returns hipSuccess or the launch error.
hipError_t launch(Kind kind, const rs_layer& layer, const StepParams& p, hipStream_t stream);

}  // namespace rs
