// ps_stubs.cpp - entry points declared in ps.h whose device paths are not
// built yet: they validate nothing and report PS_ERR_UNSUPPORTED.
#include "ps_internal.h"

using namespace ps;

extern "C" {

ps_status ps_offload_plan_create(const ps_offload_group*, int32_t, ps_offload_plan** plan) {
  if (plan) *plan = nullptr;
  return fail(PS_ERR_UNSUPPORTED, "offload pipeline not available in this build");
}

ps_status ps_offload_run(ps_offload_plan*, const ps_hparams*, int64_t, ps_stream_t) {
  return fail(PS_ERR_UNSUPPORTED, "offload pipeline not available in this build");
}

ps_status ps_offload_bytes(const ps_offload_plan*, uint64_t*, uint64_t*) {
  return fail(PS_ERR_UNSUPPORTED, "offload pipeline not available in this build");
}

ps_status ps_offload_plan_destroy(ps_offload_plan*) { return PS_OK; }

}  // extern "C"
