// ska_rdr.h -- shared between the host library and the RDR kernel unit.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ska {

struct RdrArgs {
    const float *u;          // [B][max_states] utility of each state
    const float *knorm;      // [B][max_states] key magnitude of each state
    const uint8_t *prot;     // [B][max_states] protected (non-zero)
    const int32_t *nstate;   // [B] states of each sequence
    const int64_t *budget;   // [B] byte budget of each sequence
    int max_states;
    int ntiers;
    int tiers[8];            // increasing widths
    double eps[8];           // angular error of each tier
    int64_t bytes[8];        // bytes of one retained state at each tier (non-decreasing)
    double sigma;
    uint8_t *tier_out;       // [B][max_states] 0 = evicted, else the tier
    int32_t *page_out;       // [B][max_states] page of each retained state (-1: evicted)
    int32_t *slot_out;       // [B][max_states] slot in its page (-1: evicted)
    uint8_t *page_tier;      // [B][max_pages_out] tier of each page
    int max_pages_out;
    int32_t *npages;         // [B]
    double *lambda;          // [B] the multiplier of the plan
    int32_t *status;         // [B] 0, or 2: protected states alone over the budget
    // workspace: per sequence the bound's bit pattern, the byte totals of each
    // round ([17][16]), the interval of each round ([17][2]) and per chunk the
    // count of each tier ([nchunk][8]); ws_hib and ws_tot zero on entry
    unsigned long long *ws_hib;   // [B]
    long long *ws_tot;            // [B][17][16]
    double *ws_iv;                // [B][17][2]
    int32_t *ws_cnt;              // [B][nchunk][8]
    int nchunk;                   // chunks of rdr_chunk_states() states per sequence
};

hipError_t launch_rdr(const RdrArgs &a, int batch, hipStream_t s);
int rdr_chunk_states();

}  // namespace ska
