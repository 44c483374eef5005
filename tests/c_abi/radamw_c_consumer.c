/*
 * A plain C99 consumer of include/radamw.h and libradamw.so: the header
 * compiles as strict C, the library links from C, and the entry points
 * that need no device answer from C as they do through the Python binding.
 * Built and run by the host test suite; it makes no HIP call itself and
 * calls only library functions that return before touching a device.
 *
 * Output (one "name value" pair per line) is parsed by the test.
 */
#include <stdint.h>
#include <stdio.h>

#include "radamw.h"

int main(void)
{
    radamw_options o = radamw_options_default();
    printf("lr %.17g\nbeta1 %.17g\nbeta2 %.17g\neps %.17g\nweight_decay %.17g\namsgrad %d\nmaximize %d\n",
           o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, (int)o.amsgrad, (int)o.maximize);

    /* the merge plan at the pages' largest row count */
    int64_t scratch = -1;
    int32_t extra = -1;
    int rc = radamw_stats_plan(4194304, &scratch, &extra);
    printf("plan_rc %d\nplan_scratch_elements %lld\nplan_extra_merge_kernels %d\n", rc, (long long)scratch,
           (int)extra);
    printf("plan_out_of_range %d\n", radamw_stats_plan(4194305, &scratch, &extra));

    /* the FP32 coefficients of update t = 1000 with a loss scale of 128 */
    float c[9];
    rc = radamw_host_coefficients(&o, 1000, 128.0, c);
    printf("coef_rc %d\n", rc);
    for (int i = 0; i < 9; ++i)
        printf("coef%d %.9g\n", i, (double)c[i]);

    /* a skipped step and an invalid one are answered before any device work */
    radamw_state st = {7, NULL, NULL, NULL};
    radamw_control skip = {1.0, 1};
    int32_t updated = -1;
    rc = radamw_step_inplace(NULL, NULL, RADAMW_F32, 0, &st, &o, &skip, NULL, &updated);
    printf("empty_rc %d\nempty_updated %d\nempty_step %llu\n", rc, (int)updated, (unsigned long long)st.step);
    radamw_control bad = {0.0, 0};
    printf("bad_scale_rc %d\n", radamw_step_inplace(NULL, NULL, RADAMW_F32, 16, &st, &o, &bad, NULL, &updated));
    printf("status_alias %s\n", radamw_status_string(RADAMW_ERR_ALIAS));
    printf("launches %llu\n", (unsigned long long)radamw_launch_count());
    return 0;
}
