// Internal interface between the C-ABI layer (pk_api.cpp) and the ring-attention kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pk.h"

namespace pk {

// Ring-attention local share (head dimension 128): queries of every (batch, head) against the
// key/value chunks in order first_chunk, first_chunk+1, ... (mod num_chunks).
struct AttnArgs {
    int64_t BH, Sq, chunk_len;
    int num_chunks, first_chunk;
    const uint16_t* Q;
    int64_t q_bh, ldq;
    const uint16_t* K[PK_MAX_PARTS];
    const uint16_t* V[PK_MAX_PARTS];
    int64_t k_bh, ldk, v_bh, ldv;
    float scale_log2;  // softmax scale times log2(e)
    void* O;
    int64_t o_bh, ldo;
    int o_f32;
    int split_probs;   // carry the probabilities as two bf16 terms (hi + lo)
    float* lse;        // may be null
    int64_t lse_bh;
};
hipError_t launch_ring_attention(const AttnArgs& a, hipStream_t stream);
int ring_attention_block_keys();  // chunk_len must be a multiple of this
int ring_attention_head_dim();

}  // namespace pk
