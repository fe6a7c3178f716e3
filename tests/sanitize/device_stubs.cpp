// Host-only stand-ins for the device launchers, linked into the sanitizer
// build of the library's host code (argument validation, table builder).
// Each reports that this build has no device; nothing here runs a kernel.
#include "segkv_internal.h"

namespace segkv {
namespace {
int no_device(const char *what) { return fail(SEGKV_ERR_UNSUPPORTED, "%s: host-only build", what); }
}  // namespace

int launch_write_pages(const segkv_config &, const void *, const void *, int64_t, const int32_t *, const int32_t *,
                       const int32_t *, int32_t, int32_t, int32_t, void *)
{
    return no_device("write_pages");
}
int launch_gather_pages(const segkv_config &, const int32_t *, int64_t, void *, void *, void *)
{
    return no_device("gather_pages");
}
int launch_rope_realign(const segkv_config &, const int32_t *, int64_t, float, void *)
{
    return no_device("rope_realign");
}
int launch_select_tokens(const float *, const int32_t *, const int32_t *, const int32_t *, int32_t, int64_t,
                         int32_t *, void *)
{
    return no_device("select_tokens");
}
int launch_sparse_ffn(void *, int64_t, int32_t, int32_t, const int32_t *, int32_t, const void *, const void *,
                      const void *, void *, void *)
{
    return no_device("sparse_ffn");
}
int launch_attn_mass(const segkv_config &, const segkv_dev_tables &, const void *, const float *, float, float *,
                     void *)
{
    return no_device("attn_mass");
}
int launch_attn_prefill(const segkv_config &, const segkv_dev_tables &, const void *, void *, int32_t, float *, float,
                        void *, void *)
{
    return no_device("attn_prefill");
}
int noalloc_scratch(void **out)
{
    *out = nullptr;
    return no_device("attn_prefill_noalloc");
}

}  // namespace segkv
