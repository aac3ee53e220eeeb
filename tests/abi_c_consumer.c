/* A plain C99 consumer of include/sage_attn.h: host-only calls (no device work), built with
 * gcc -std=c99 -pedantic against the in-tree library by tests/test_abi_c_consumer.py. */
#include <stdio.h>
#include <string.h>

#include "sage_attn.h"

static int fails = 0;
#define CHECK(c)                                           \
    do {                                                   \
        if (!(c)) {                                        \
            printf("FAIL line %d: %s\n", __LINE__, #c);    \
            fails++;                                       \
        }                                                  \
    } while (0)

int main(void)
{
    sage_problem p;
    sage_quant_layout L;
    sage_varlen_problem vp;
    size_t bytes = 0, bwd = 0, vbytes = 0;

    CHECK(sage_abi_version() == SAGE_ABI_VERSION);
    CHECK(strcmp(sage_status_string(SAGE_OK), "ok") == 0);
    CHECK(strlen(sage_status_string(SAGE_ERR_WORKSPACE)) > 0);

    /* the headline problem: B=1 H=32 N=4096 d=128, causal, INT8 QK / FP8 P~V */
    memset(&p, 0, sizeof p);
    p.B = 1; p.H = 32; p.N = 4096; p.d = 128; p.causal = 1; p.sm_scale = 0.08838834764f;
    p.io_dtype = SAGE_DT_BF16; p.qk_fmt = SAGE_FMT_INT8; p.pv_fmt = SAGE_FMT_FP8;
    CHECK(sage_quant_size(&p, &bytes, &L) == SAGE_OK);
    CHECK(bytes == L.total && bytes > 0);
    /* every part lies inside the buffer, 256-byte aligned, in the documented order */
    CHECK(L.mu_k % 256 == 0 && L.mu_k < L.mu_q && L.mu_q < L.q_codes && L.q_codes < L.q_scales);
    CHECK(L.q_scales < L.k_codes && L.k_codes < L.k_scales && L.k_scales < L.v_codes);
    CHECK(L.v_codes < L.v_scales && L.v_scales < L.delta_s && L.delta_s < L.lse_corr && L.lse_corr < L.stats);
    CHECK(L.stats < L.total);
    /* INT8 codes: at least one byte per element of Q and K, and of V */
    CHECK(L.k_codes - L.q_codes >= (size_t)32 * 4096 * 128);
    CHECK(sage_attn_bwd_ws_size(&p, &bwd) == SAGE_OK && bwd > bytes);

    /* an unsupported head dimension: UNSUPPORTED with a message, outputs untouched */
    p.d = 96;
    bytes = 12345;
    CHECK(sage_quant_size(&p, &bytes, NULL) == SAGE_ERR_UNSUPPORTED);
    CHECK(bytes == 12345 && strlen(sage_last_error()) > 0);
    p.d = 128;
    /* a NULL tensor pointer is rejected before anything is launched */
    CHECK(sage_attn_fwd(NULL, NULL, NULL, NULL, 1, 32, 4096, 128, 1, 0.088f, SAGE_FMT_INT8, SAGE_FMT_FP8, NULL) ==
          SAGE_ERR_INVALID_ARG);

    /* packed sequences with grouped KV heads and per-block Q smoothing */
    memset(&vp, 0, sizeof vp);
    vp.B = 3; vp.H = 8; vp.H_kv = 2; vp.d = 64; vp.causal = 0; vp.sm_scale = 0.125f;
    vp.io_dtype = SAGE_DT_F16; vp.qk_fmt = SAGE_FMT_MXFP4_QBLOCK; vp.pv_fmt = SAGE_FMT_FP8;
    vp.total_q = 900; vp.total_k = 700; vp.max_seqlen_q = 500; vp.max_seqlen_k = 400;
    CHECK(sage_varlen_ws_size(&vp, &vbytes) == SAGE_OK && vbytes > 0);
    vp.H_kv = 3;   /* 8 query heads cannot share 3 KV heads */
    CHECK(sage_varlen_ws_size(&vp, &vbytes) == SAGE_ERR_INVALID_ARG);

    if (fails == 0)
        printf("abi c consumer ok\n");
    return fails != 0;
}
