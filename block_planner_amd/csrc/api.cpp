// api.cpp -- host-only parts of the C ABI (no GPU work).
#include "../../include/ht.h"

extern "C" const char *ht_status_string(ht_status s) {
    switch (s) {
    case HT_OK: return "ok";
    case HT_EINVAL: return "invalid argument";
    case HT_ESHAPE: return "invalid shape";
    case HT_EALIGN: return "misaligned pointer or stride";
    case HT_ESMALL: return "buffer or workspace too small";
    case HT_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

// Defaults: eps_int4 0.08, eps_int8 0.01; eps_bf16 = eps_fp16 = 0 and
// prefer_bf16 = 1 as in the HyperTensor page's "Convert model" call.
extern "C" void ht_plan_params_default(ht_plan_params *p) {
    if (!p) return;
    p->eps_int4 = 0.08;
    p->eps_int8 = 0.01;
    p->eps_bf16 = 0.0;
    p->eps_fp16 = 0.0;
    p->prefer_bf16 = 1;
    p->force_format = -1;
}
