// qs_attn_gqa.hip -- the attention and combine kernels of one call variant: grouped queries (qs_attend_draft_gqa / qs_attend_verify_gqa).
#include "qs_device.h"

namespace qs {

hipError_t launch_attention_gqa(const AttnGqaArgs& a, int D, bool draft, hipStream_t st) {
  return launch_attention_m<kModeGqa>(a, D, draft, st);
}

const void* attn_fn_gqa(int D, bool draft, int bucket, bool meta16, bool pair) {
  if (pair) return meta16 ? attn_fn_gqa_pair<true>(D, bucket) : attn_fn_gqa_pair<false>(D, bucket);
  return meta16 ? attn_fn_dm<kModeGqa, true>(D, draft, bucket) : attn_fn_dm<kModeGqa, false>(D, draft, bucket);
}

}  // namespace qs
